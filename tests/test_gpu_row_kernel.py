"""The one-row QMV kernel: 16-bit x against MXFP4, NVFP4 or MXFP8 weights
with K = 2048 or 4096 (qmv_row_kernel), at one to four activation rows.

Each activation row is folded exactly as a one-row call folds it, so every
batch row of a call the kernel takes (bf16: B <= 2 for MXFP4, <= 3 for NVFP4,
<= 4 for MXFP8; f16: B <= 4) must equal the one-row call of that row bit for
bit. The kernel shares the per-unit arithmetic and the reduction order with
the VALU tile, which f16 calls of six NVFP4 or MXFP8 rows run (f16 MXFP4
batches go from the one-row kernel straight to the matrix cores at B = 5; the
gather tests pin those rows to the same arithmetic): their rows must equal the
one-row calls bit for bit too. Every case is
also checked against the fp64 oracle on sampled rows. The cases cover ragged N
(the last block's rows past N re-read row N - 1 and are not stored), a single
row, NVFP4 with and without its global scale, and rows whose scales take the
end codes of their formats (E8M0 0, 1, 2 and the NaN code; E4M3 block scales
0x00, 0x01, 0x08, 0x7E and the NaN code).
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


def _case(fmt, dtype, K, N, key, gscale=0.5, exp_range=(120, 130), B=2):
    if fmt == "mxfp4":
        return workloads.mxfp4_case(75, key, K=K, N=N, B=B, dtype=dtype, exp_range=exp_range)
    if fmt == "mxfp8":
        return workloads.mxfp8_case(75, key, K=K, N=N, B=B, dtype=dtype, exp_range=exp_range)
    return workloads.nvfp4_case(75, key, K=K, N=N, B=B, dtype=dtype, global_scale=gscale)


def _bits(y, dtype):
    return y.view(np.uint16) if dtype in ("bf16", "f16") else y.view(np.uint32)


# activation rows the one-row kernel takes, per (dtype, format)
ROW_MAX = {("bf16", "mxfp4"): 2, ("bf16", "nvfp4"): 3, ("bf16", "mxfp8"): 4,
           ("f16", "mxfp4"): 4, ("f16", "nvfp4"): 4, ("f16", "mxfp8"): 4}


def _one_row_calls(bmv, c):
    """[B, N] output of one-row calls, one per activation row of case c."""
    out = []
    for b in range(c.B):
        cb = dataclasses.replace(c, B=1, x=c.x[b:b + 1].copy())
        out.append(to_host(run_qmv(bmv, cb), c.dtype)[0])
    return np.stack(out)


def _check_batches(bmv, c6, what):
    """c6 has six activation rows. Every call of 2..ROW_MAX rows equals the
    one-row calls bit for bit; for f16 NVFP4 / MXFP8 so does the six-row call
    (the VALU tile). Returns (the one-row case of row 0, one-row outputs
    [6, N])."""
    dtype = c6.dtype
    y1 = _one_row_calls(bmv, c6)
    top = ROW_MAX[(dtype, c6.fmt)]
    for B in range(2, top + 1):
        cb = dataclasses.replace(c6, B=B, x=c6.x[:B].copy())
        yb = to_host(run_qmv(bmv, cb), dtype)
        assert np.array_equal(_bits(yb, dtype), _bits(y1[:B], dtype)), \
            f"{what}: a row of the {B}-row call differs from its one-row call"
    if dtype == "f16" and c6.fmt != "mxfp4":
        y6 = to_host(run_qmv(bmv, c6), dtype)
        assert np.array_equal(_bits(y6, dtype), _bits(y1, dtype)), \
            f"{what}: the VALU tile's rows differ from the one-row kernel's"
    return dataclasses.replace(c6, B=1, x=c6.x[:1].copy()), y1


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(2048, 301), (4096, 1), (4096, 9), (4096, 2051)])
def test_row_kernel_equals_tile_and_oracle(bmv, fmt, dtype, K, N):
    # f16 outputs of MXFP8 rows with E8M0 up to 2^3 pass 65504 at K=4096
    er = (116, 126) if (fmt, dtype) == ("mxfp8", "f16") else (120, 130)
    c6 = _case(fmt, dtype, K, N, f"row-{fmt}-{dtype}-{K}-{N}", exp_range=er, B=6)
    say(f"row kernel {fmt} {dtype} K={K} N={N}")
    c1, y1 = _check_batches(bmv, c6, f"{fmt} {dtype} K={K} N={N}")
    rows = sample_rows(N, 64, seed=K + N)
    y64, A = oracle_rows(c1, rows)
    check(y1[:1, rows], y64, A, dtype, f"row kernel {fmt} {dtype} K={K} N={N}")
    # the last row of the widest call the kernel takes, against the oracle too
    top = ROW_MAX[(dtype, fmt)]
    cl = dataclasses.replace(c6, B=1, x=c6.x[top - 1:top].copy())
    y64, A = oracle_rows(cl, rows)
    check(y1[top - 1:top, rows], y64, A, dtype, f"row kernel {fmt} {dtype} K={K} N={N} row {top - 1}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_kernel_nvfp4_without_global_scale(bmv, dtype):
    c6 = _case("nvfp4", dtype, 4096, 77, f"row-nvfp4-nogs-{dtype}", gscale=None, B=6)
    say(f"row kernel nvfp4 without global scale {dtype}")
    c1, y1 = _check_batches(bmv, c6, f"nvfp4 no global scale {dtype}")
    rows = np.arange(77)
    y64, A = oracle_rows(c1, rows)
    check(y1[:1], y64, A, dtype, f"row kernel nvfp4 no global scale {dtype}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K", [2048, 4096])
def test_row_kernel_extreme_scale_codes(bmv, fmt, dtype, K):
    c6 = _case(fmt, dtype, K, 24, f"row-extreme-{fmt}-{dtype}-{K}", B=6)
    sc = c6.scales.copy()
    if fmt == "nvfp4":
        sc[0, :] = 0x01
        sc[1, ::2] = 0x00
        sc[2, :] = 0x08
        sc[3, 5] = 0x7F               # NaN block
        # the largest code; f16 outputs of K=4096 rows would overflow with it
        sc[4, :] = 0x7E if dtype == "bf16" else 0x66
    else:
        sc[0, :] = 0
        sc[1, :] = 1
        sc[2, ::2] = 2
        sc[3, 7] = 255                # NaN block
        sc[4, :] = np.where(np.arange(sc.shape[1]) % 2 == 0, 0, 130 if dtype == "bf16" else 118)
    c6.scales = sc
    say(f"row kernel extreme scale codes {fmt} {dtype} K={K}")
    c1, y1 = _check_batches(bmv, c6, f"extreme scales {fmt} {dtype} K={K}")
    assert np.isnan(oracle.storage_to_f64(y1[:, [3]], dtype)).all()
    keep = np.setdiff1d(np.arange(c1.N), [3])
    y64, A = oracle_rows(c1, keep)
    check(y1[:1, keep], y64, A, dtype, f"row kernel extreme scales {fmt} {dtype} K={K}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(2048, 77), (4096, 301)])
def test_row_norm_kernel_equals_tile_and_definition(bmv, fmt, dtype, K, N):
    """The fused RMSNorm + QMV on the one-row kernel (with the norm accessor):
    every call of 2..ROW_MAX rows equals the one-row calls bit for bit (r
    included), for f16 MXFP8 so does the five-row call (the fused VALU tile;
    f16 MXFP4 and NVFP4 take the matrix cores from five rows), and the
    one-row calls meet the plain fp64 definition W . rmsnorm(x) within the
    staging bound."""
    from gpu_util import case_to_dev, check_fused_norm, to_dev
    # the normalized row has unit RMS whatever x's scale, so the outputs'
    # size is the weights'; E8M0 scales of 2^-13 .. 2^-3 keep every f16 output
    # finite (with scales up to 2^3, MXFP8 rows of K=4096 overflow f16)
    c5 = _case(fmt, dtype, K, N, f"rownorm-{fmt}-{dtype}-{K}-{N}", exp_range=(114, 124),
                       B=5)
    rng = workloads.rng_for(76, f"gamma-{fmt}-{dtype}-{K}")
    gamma = workloads.to_storage(rng.uniform(0.5, 1.5, size=K), dtype)
    x5 = workloads.to_storage(oracle.storage_to_f64(c5.x, dtype) * 3.0, dtype)
    d = case_to_dev(c5)
    blk = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, d["w"], d["scales"], None, K=K, bits=c5.bits, group_size=blk,
                          global_scale=d.get("gscale"))
    eps = 1e-6
    say(f"row norm kernel {fmt} {dtype} K={K} N={N}")

    def call(x):
        return to_host(bmv.qmv_rmsnorm_qmv(to_dev(x.copy(), dtype), wt, to_dev(gamma, dtype), eps),
                       dtype)

    y1 = np.stack([call(x5[b:b + 1])[0] for b in range(5)])
    top = ROW_MAX[(dtype, fmt)]
    for B in range(2, top + 1):
        assert np.array_equal(_bits(call(x5[:B]), dtype), _bits(y1[:B], dtype)), \
            f"{fmt} {dtype} K={K}: a row of the {B}-row fused call differs from its one-row call"
    if dtype == "f16" and fmt == "mxfp8":
        assert np.array_equal(_bits(call(x5), dtype), _bits(y1, dtype)), \
            f"{fmt} {dtype} K={K}: the fused VALU tile's rows differ from the one-row kernel's"
    W = oracle.dequant(fmt, K, c5.w, c5.scales, None, bits=c5.bits, group=c5.group, dtype=dtype,
                       global_scale=c5.global_scale)
    for b in (0, top - 1):
        y_def = oracle.rmsnorm_qmv(x5[b:b + 1], dtype, gamma, eps, W)
        A_def = oracle.rmsnorm_qmv_abs(x5[b:b + 1], dtype, gamma, eps, W)
        check_fused_norm(y1[b:b + 1], y_def, A_def, dtype,
                         f"row norm kernel {fmt} {dtype} K={K} N={N} row {b}")


# ---------------------------------------------------------------------------
# 4-bit affine codes with 16-bit x (groups of 32, 64 and 128) on the one-row
# kernel at B <= 4; affine never takes the matrix cores, so a five-row call
# runs the VALU tile, whose rows must equal the one-row calls bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(2048, 77), (4096, 301)])
def test_row_kernel_affine4(bmv, group, dtype, K, N):
    c = workloads.affine_case(75, f"row-aff-{group}-{dtype}-{K}-{N}", bits=4, group=group, K=K,
                              N=N, B=5, dtype=dtype)
    say(f"row kernel affine 4-bit g{group} {dtype} K={K} N={N}")
    y1 = _one_row_calls(bmv, c)
    for B in range(2, 6):
        yb = to_host(run_qmv(bmv, dataclasses.replace(c, B=B, x=c.x[:B].copy())), dtype)
        assert np.array_equal(_bits(yb, dtype), _bits(y1[:B], dtype)), \
            f"affine g{group} {dtype} K={K}: a row of the {B}-row call differs from its one-row call"
    rows = sample_rows(N, 64, seed=K + N + group)
    for b in (0, 3):
        cb = dataclasses.replace(c, B=1, x=c.x[b:b + 1].copy())
        y64, A = oracle_rows(cb, rows)
        check(y1[b:b + 1, rows], y64, A, dtype, f"row kernel affine g{group} {dtype} K={K} row {b}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_norm_kernel_affine4(bmv, dtype):
    """The fused RMSNorm + QMV of 4-bit affine codes on the one-row kernel:
    batch rows equal one-row calls bit for bit up to B = 4 and so do the
    fused VALU tile's rows at B = 5; the one-row calls meet the plain
    definition within the staging bound."""
    from gpu_util import case_to_dev, check_fused_norm, to_dev
    K, N = 4096, 301
    c = workloads.affine_case(75, f"rownorm-aff-{dtype}", bits=4, group=64, K=K, N=N, B=5,
                              dtype=dtype)
    gamma = workloads.to_storage(workloads.rng_for(76, f"gamma-aff-{dtype}").uniform(0.5, 1.5, size=K),
                                 dtype)
    x5 = workloads.to_storage(oracle.storage_to_f64(c.x, dtype) * 3.0, dtype)
    d = case_to_dev(c)
    wt = bmv.make_weights("affine", d["w"], d["scales"], d["biases"], K=K, bits=4, group_size=64)
    say(f"row norm kernel affine 4-bit g64 {dtype} K={K} N={N}")

    def call(x):
        return to_host(bmv.qmv_rmsnorm_qmv(to_dev(x.copy(), dtype), wt, to_dev(gamma, dtype), 1e-6),
                       dtype)

    y1 = np.stack([call(x5[b:b + 1])[0] for b in range(5)])
    for B in range(2, 6):
        assert np.array_equal(_bits(call(x5[:B]), dtype), _bits(y1[:B], dtype)), \
            f"affine {dtype}: a row of the {B}-row fused call differs from its one-row call"
    W = oracle.dequant("affine", K, c.w, c.scales, c.biases, bits=4, group=64, dtype=dtype)
    y_def = oracle.rmsnorm_qmv(x5[:1], dtype, gamma, 1e-6, W)
    A_def = oracle.rmsnorm_qmv_abs(x5[:1], dtype, gamma, 1e-6, W)
    check_fused_norm(y1[:1], y_def, A_def, dtype, f"row norm kernel affine {dtype}")
