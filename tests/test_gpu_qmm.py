"""GPU parity of qmm (y = x . W^T for M rows, matrix cores) against the
oracle, with the QMV parity bar (A = sum_k |x[m, k] W[n, k]|)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import case_to_dev, check, oracle_rows, sample_rows, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _case(fmt, bits, group, M, K, N, dtype, key):
    if fmt == "affine":
        return workloads.affine_case(9, key, bits=bits, group=group, K=K, N=N, B=M, dtype=dtype)
    if fmt == "mxfp4":
        return workloads.mxfp4_case(9, key, K=K, N=N, B=M, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(9, key, K=K, N=N, B=M, dtype=dtype)
    return workloads.mxfp8_case(9, key, K=K, N=N, B=M, dtype=dtype)


def _run(bmv, c):
    d = case_to_dev(c)
    blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
    wt = bmv.make_weights(c.fmt, d["w"], d["scales"], d.get("biases"), K=c.K, bits=c.bits,
                          group_size=blk, global_scale=d.get("gscale"))
    return bmv.qmv_qmm(d["x"], wt), wt, d


AFFINE = [("affine", b, g) for b in (2, 3, 4, 5, 6, 8) for g in (32, 64, 128)]
FP = [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)]


@pytest.mark.parametrize("fmt,bits,group", AFFINE + FP)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_qmm_ragged(bmv, fmt, bits, group, dtype):
    # M below one tile and past one, N ragged against the 128-column tile,
    # K with a half slice at the end (K % 64 == 32) where the group allows it
    K = {32: 1056, 16: 1056, 64: 1088, 128: 1152}[group]
    for M in (9, 70):
        key = f"{fmt}-{bits}-{group}-{dtype}-{M}"
        say(f"qmm {key} M={M} N=300 K={K}")
        c = _case(fmt, bits, group, M, K, 300, dtype, key)
        y, _, _ = _run(bmv, c)
        y64, A = oracle_rows(c, np.arange(c.N))
        check(to_host(y, dtype), y64, A, dtype, f"qmm {key}")


@pytest.mark.parametrize("fmt,bits,group", [("affine", 4, 64), ("mxfp4", 4, 32),
                                            ("nvfp4", 4, 16), ("mxfp8", 8, 32)])
def test_qmm_full_size_sampled(bmv, fmt, bits, group):
    # M = 256 rows against the K = 4096, N = 14336 matrix, sampled columns
    key = f"{fmt}-full"
    say(f"qmm {key} bf16 M=256 K=4096 N=14336 sampled columns")
    c = _case(fmt, bits, group, 256, 4096, 14336, "bf16", key)
    y, _, _ = _run(bmv, c)
    cols = sample_rows(c.N, 48)
    y64, A = oracle_rows(c, cols)
    check(to_host(y, "bf16")[:, cols], y64, A, "bf16", f"qmm {key}")


def test_qmm_rows_match_qmv(bmv):
    # at M = 8 both the qmm and the QMV meet the bar against the same oracle
    import torch
    say("qmm vs qmv mxfp4 bf16 M=8 K=2048 N=512")
    c = _case("mxfp4", 4, 32, 8, 2048, 512, "bf16", "vs-qmv")
    y, wt, d = _run(bmv, c)
    y8 = bmv.qmv_fp_mxfp4(d["x"], d["w"], d["scales"])
    y64, A = oracle_rows(c, np.arange(c.N))
    check(to_host(y, "bf16"), y64, A, "bf16", "qmm M=8")
    torch.cuda.synchronize()
    check(to_host(y8, "bf16"), y64, A, "bf16", "qmv M=8")


def test_qmm_k_zero_and_m_one(bmv):
    import torch
    say("qmm affine 4b g64 bf16 M=1 K=512 N=130")
    c = _case("affine", 4, 64, 1, 512, 130, "bf16", "m1")
    y, _, _ = _run(bmv, c)
    y64, A = oracle_rows(c, np.arange(c.N))
    check(to_host(y, "bf16"), y64, A, "bf16", "qmm M=1")
    # K == 0: empty sums
    wt = bmv.make_weights("mxfp4", torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"),
                          torch.zeros((5, 0), dtype=torch.uint8, device="cuda:0"), K=0)
    x = torch.zeros((12, 0), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((12, 5), 7.0, dtype=torch.bfloat16, device="cuda:0")
    bmv.qmv_qmm(x, wt, y=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_qmm_repeatable(bmv):
    import torch
    say("qmm nvfp4 f16 M=96 K=1024 N=640, twice")
    c = _case("nvfp4", 4, 16, 96, 1024, 640, "f16", "rep")
    y, wt, d = _run(bmv, c)
    y2 = bmv.qmv_qmm(d["x"], wt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
