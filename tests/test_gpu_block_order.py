"""The XCD-chunked block order of the QMV kernels, on every output row.

The one-row kernel, the VALU tile and their fused-RMSNorm forms reorder each
group of 64 consecutive blocks so that the eight blocks an XCD receives own
consecutive row tiles; blocks past the last whole group keep their index.
Small grids (under 64 blocks) never reorder, so these cases use grids of
several whole groups plus a partial one, write into an output pre-filled with
NaN (a row no block wrote, or one written twice with the wrong data, shows),
and check every row against the fp64 oracle.
"""
from __future__ import annotations

import numpy as np
import oracle
import pytest

import workloads
from gpu_util import case_to_dev, check, check_fused_norm, oracle_rows, run_qmv, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _nan_out(c):
    import torch
    from gpu_util import torch_dtype
    return torch.full((c.B, c.N), float("nan"), dtype=torch_dtype(c.dtype), device="cuda:0")


def _case(fmt, dtype, B, K, N, key):
    if fmt == "mxfp4":
        return workloads.mxfp4_case(78, key, K=K, N=N, B=B, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(78, key, K=K, N=N, B=B, dtype=dtype, global_scale=0.5)
    if fmt == "mxfp8":
        return workloads.mxfp8_case(78, key, K=K, N=N, B=B, dtype=dtype)
    return workloads.affine_case(78, key, bits=4, group=64, K=K, N=N, B=B, dtype=dtype)


# (format, dtype, B, K, N): the one-row kernel takes 8 rows per block at one to
# four activation rows (N=2051: 257 blocks = 4 whole groups + 1; N=1100: 138
# blocks), the VALU tile
# 4 (64 / LPR) R rows per block: 4 for K = 4096 at B <= 2 (N=1100: 275
# blocks), 32 for the 16-lane rows of K = 1536 at B = 3 (N=2200: 69 blocks)
CASES = [
    ("mxfp4", "bf16", 1, 4096, 2051),
    ("nvfp4", "f16", 1, 4096, 2051),
    ("mxfp8", "bf16", 1, 2048, 1100),
    ("affine", "bf16", 1, 4096, 1100),
    ("affine", "f32", 2, 4096, 1100),
    ("mxfp4", "f16", 3, 1536, 2200),
    ("mxfp4", "f16", 2, 4096, 1100),
    ("nvfp4", "bf16", 3, 4096, 2051),
    ("mxfp8", "bf16", 4, 2048, 1100),
]


@pytest.mark.parametrize("fmt,dtype,B,K,N", CASES)
def test_block_order_every_row(bmv, fmt, dtype, B, K, N):
    c = _case(fmt, dtype, B, K, N, f"order-{fmt}-{dtype}-{B}-{K}-{N}")
    say(f"block order {fmt} {dtype} B={B} K={K} N={N}: all rows")
    y = to_host(run_qmv(bmv, c, y=_nan_out(c)), dtype)
    y64, A = oracle_rows(c, np.arange(N))
    check(y, y64, A, dtype, f"block order {fmt} {dtype} B={B} K={K} N={N}")


@pytest.mark.parametrize("fmt,dtype,B,K,N", [("mxfp4", "bf16", 1, 4096, 2051),
                                             ("affine", "f16", 1, 4096, 1100),
                                             ("nvfp4", "bf16", 3, 4096, 2051)])
def test_block_order_fused_norm_every_row(bmv, fmt, dtype, B, K, N):
    c = _case(fmt, dtype, B, K, N, f"order-norm-{fmt}-{dtype}-{K}-{N}")
    say(f"block order fused RMSNorm {fmt} {dtype} B={B} K={K} N={N}: all rows")
    rng = workloads.rng_for(78, f"order-gamma-{fmt}-{dtype}")
    gamma = workloads.to_storage(rng.uniform(0.5, 1.5, size=K), dtype)
    d = case_to_dev(c)
    blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[fmt]
    wt = bmv.make_weights(fmt, d["w"], d["scales"], d.get("biases"), K=K, bits=c.bits,
                          group_size=blk, global_scale=d.get("gscale"))
    eps = 1e-6
    y = to_host(bmv.qmv_rmsnorm_qmv(d["x"], wt, to_dev(gamma, dtype), eps, y=_nan_out(c)), dtype)
    W = oracle.dequant(fmt, K, c.w, c.scales, c.biases, bits=c.bits, group=c.group, dtype=dtype,
                       global_scale=c.global_scale)
    y_def = oracle.rmsnorm_qmv(c.x, dtype, gamma, eps, W)
    A_def = oracle.rmsnorm_qmv_abs(c.x, dtype, gamma, eps, W)
    check_fused_norm(y, y_def, A_def, dtype, f"block order fused norm {fmt} {dtype} N={N}")
