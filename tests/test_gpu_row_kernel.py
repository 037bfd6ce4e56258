"""The one-activation-row QMV kernel: 16-bit x against MXFP4, NVFP4 or MXFP8
weights with K = 2048 or 4096 (qmv_row_kernel).

Every case is checked twice: against the fp64 oracle on sampled rows, and bit
for bit against the same activation row computed by the VALU tile, which is
what a two-row call of the same weights runs (below the matrix-core
thresholds). The two kernels share the per-unit arithmetic and the reduction
order, so a row's result must not depend on which of them computed it. The
cases cover ragged N (the last block's rows past N re-read row N - 1 and are
not stored), a single row, NVFP4 with and without its global scale, and rows
whose scales take the end codes of their formats (E8M0 0, 1, 2 and the NaN
code; E4M3 block scales 0x00, 0x01, 0x08, 0x7E and the NaN code).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import oracle
import pytest

import workloads
from gpu_util import check, oracle_rows, run_qmv, sample_rows, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _two_row_case(fmt, dtype, K, N, key, gscale=0.5, exp_range=(120, 130)):
    if fmt == "mxfp4":
        return workloads.mxfp4_case(75, key, K=K, N=N, B=2, dtype=dtype, exp_range=exp_range)
    if fmt == "mxfp8":
        return workloads.mxfp8_case(75, key, K=K, N=N, B=2, dtype=dtype, exp_range=exp_range)
    return workloads.nvfp4_case(75, key, K=K, N=N, B=2, dtype=dtype, global_scale=gscale)


def _bits(y, dtype):
    return y.view(np.uint16) if dtype in ("bf16", "f16") else y.view(np.uint32)


def _row_and_tile(bmv, c2):
    """(B=1 output [1, N], B=2 output [2, N]) for the case's first x row."""
    c1 = dataclasses.replace(c2, B=1, x=c2.x[:1].copy())
    y1 = to_host(run_qmv(bmv, c1), c1.dtype)
    y2 = to_host(run_qmv(bmv, c2), c2.dtype)
    return c1, y1, y2


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(2048, 301), (4096, 1), (4096, 9), (4096, 2051)])
def test_row_kernel_equals_tile_and_oracle(bmv, fmt, dtype, K, N):
    c2 = _two_row_case(fmt, dtype, K, N, f"row-{fmt}-{dtype}-{K}-{N}")
    say(f"row kernel {fmt} {dtype} K={K} N={N}")
    c1, y1, y2 = _row_and_tile(bmv, c2)
    assert np.array_equal(_bits(y1[0], dtype), _bits(y2[0], dtype)), \
        f"{fmt} {dtype} K={K} N={N}: the one-row kernel differs from the tile's row"
    rows = sample_rows(N, 64, seed=K + N)
    y64, A = oracle_rows(c1, rows)
    check(y1[:, rows], y64, A, dtype, f"row kernel {fmt} {dtype} K={K} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_kernel_nvfp4_without_global_scale(bmv, dtype):
    c2 = _two_row_case("nvfp4", dtype, 4096, 77, f"row-nvfp4-nogs-{dtype}", gscale=None)
    say(f"row kernel nvfp4 without global scale {dtype}")
    c1, y1, y2 = _row_and_tile(bmv, c2)
    assert np.array_equal(_bits(y1[0], dtype), _bits(y2[0], dtype))
    rows = np.arange(77)
    y64, A = oracle_rows(c1, rows)
    check(y1, y64, A, dtype, f"row kernel nvfp4 no global scale {dtype}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("K", [2048, 4096])
def test_row_kernel_extreme_scale_codes(bmv, fmt, K):
    c2 = _two_row_case(fmt, "bf16", K, 24, f"row-extreme-{fmt}-{K}")
    sc = c2.scales.copy()
    if fmt == "nvfp4":
        sc[0, :] = 0x01
        sc[1, ::2] = 0x00
        sc[2, :] = 0x08
        sc[3, 5] = 0x7F               # NaN block
        sc[4, :] = 0x7E
    else:
        sc[0, :] = 0
        sc[1, :] = 1
        sc[2, ::2] = 2
        sc[3, 7] = 255                # NaN block
        sc[4, :] = np.where(np.arange(sc.shape[1]) % 2 == 0, 0, 130)
    c2.scales = sc
    say(f"row kernel extreme scale codes {fmt} K={K}")
    c1, y1, y2 = _row_and_tile(bmv, c2)
    assert np.array_equal(_bits(y1[0], "bf16"), _bits(y2[0], "bf16")), \
        f"{fmt} K={K}: the one-row kernel differs from the tile's row"
    assert np.isnan(oracle.storage_to_f64(y1[:, [3]], "bf16")).all()
    keep = np.setdiff1d(np.arange(c1.N), [3])
    y64, A = oracle_rows(c1, keep)
    check(y1[:, keep], y64, A, "bf16", f"row kernel extreme scales {fmt} K={K}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(2048, 77), (4096, 301)])
def test_row_norm_kernel_equals_tile_and_definition(bmv, fmt, dtype, K, N):
    """The fused RMSNorm + QMV at one activation row (the one-row kernel with
    the norm accessor) against the tile's row inside a two-row fused call, bit
    for bit, and against the plain fp64 definition W . rmsnorm(x) with the
    staging bound."""
    from gpu_util import case_to_dev, check_fused_norm, to_dev
    # the normalized row has unit RMS whatever x's scale, so the outputs'
    # size is the weights'; E8M0 scales of 2^-13 .. 2^-3 keep every f16 output
    # finite (with scales up to 2^3, MXFP8 rows of K=4096 overflow f16)
    c2 = _two_row_case(fmt, dtype, K, N, f"rownorm-{fmt}-{dtype}-{K}-{N}", exp_range=(114, 124))
    rng = workloads.rng_for(76, f"gamma-{fmt}-{dtype}-{K}")
    gamma = workloads.to_storage(rng.uniform(0.5, 1.5, size=K), dtype)
    x2 = workloads.to_storage(oracle.storage_to_f64(c2.x, dtype) * 3.0, dtype)
    d = case_to_dev(c2)
    blk = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, d["w"], d["scales"], None, K=K, bits=c2.bits, group_size=blk,
                          global_scale=d.get("gscale"))
    eps = 1e-6
    say(f"row norm kernel {fmt} {dtype} K={K} N={N}")
    y1 = to_host(bmv.qmv_rmsnorm_qmv(to_dev(x2[:1].copy(), dtype), wt, to_dev(gamma, dtype), eps),
                 dtype)
    y2 = to_host(bmv.qmv_rmsnorm_qmv(to_dev(x2, dtype), wt, to_dev(gamma, dtype), eps), dtype)
    assert np.array_equal(_bits(y1[0], dtype), _bits(y2[0], dtype)), \
        f"{fmt} {dtype} K={K}: the one-row fused kernel differs from the tile's row"
    W = oracle.dequant(fmt, K, c2.w, c2.scales, None, bits=c2.bits, group=c2.group, dtype=dtype,
                       global_scale=c2.global_scale)
    y_def = oracle.rmsnorm_qmv(x2[:1], dtype, gamma, eps, W)
    A_def = oracle.rmsnorm_qmv_abs(x2[:1], dtype, gamma, eps, W)
    check_fused_norm(y1, y_def, A_def, dtype, f"row norm kernel {fmt} {dtype} K={K} N={N}")
