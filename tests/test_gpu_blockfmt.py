"""GPU parity of the symmetric block-scaled formats (the rest of the Track-1
matrix): device dequant bit for bit against the oracle's fp32 rounding of the
exact product, and QMV within the parity bar, for all 27 formats."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import case_to_dev, check, oracle_rows, run_qmv, sample_rows, say, to_host

pytestmark = pytest.mark.gpu

FMTS = sorted(workloads.SB_FORMATS)


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


@pytest.mark.parametrize("fmt", FMTS)
def test_block_dequant_bit_exact(bmv, fmt):
    import torch
    say(f"dequant {fmt} N=37 K=512")
    c = workloads.sb_case(fmt, K=512, N=37, B=1, key="dq")
    d = case_to_dev(c)
    wt = bmv.make_weights(fmt, d["w"], d["scales"], K=c.K)
    out = bmv.qmv_dequant_device(wt, 2, "cuda:0")
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = oracle.dequant(fmt, c.K, c.w, c.scales).astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B", [1, 5])
def test_block_qmv(bmv, fmt, dtype, B):
    say(f"qmv {fmt} {dtype} B={B} N=300 K=512")
    c = workloads.sb_case(fmt, K=512, N=300, B=B, dtype=dtype, key="q")
    y = run_qmv(bmv, c)
    y64, A = oracle_rows(c, np.arange(c.N))
    check(to_host(y, dtype), y64, A, dtype, f"{fmt} {dtype} B={B}")


@pytest.mark.parametrize("fmt", ["nvfp8", "fp8_e5m2_f16", "int4", "mxint8", "fp4_f16"])
def test_block_qmv_f16_and_b8(bmv, fmt):
    for dtype, B in (("f16", 1), ("f16", 8), ("bf16", 8)):
        say(f"qmv {fmt} {dtype} B={B} N=200 K=1024")
        c = workloads.sb_case(fmt, K=1024, N=200, B=B, dtype=dtype, key="h")
        y = run_qmv(bmv, c)
        y64, A = oracle_rows(c, np.arange(c.N))
        check(to_host(y, dtype), y64, A, dtype, f"{fmt} {dtype} B={B}")


@pytest.mark.parametrize("fmt", ["fp8_e5m2", "int4", "mxint3", "nvfp8_f16"])
def test_block_qmv_full_size_sampled(bmv, fmt):
    say(f"qmv {fmt} bf16 B=1 K=4096 N=14336 sampled rows")
    c = workloads.sb_case(fmt, K=4096, N=14336, B=1, key="full")
    y = run_qmv(bmv, c)
    rows = sample_rows(c.N)
    y64, A = oracle_rows(c, rows)
    check(to_host(y, "bf16")[:, rows], y64, A, "bf16", f"{fmt} full size")


def test_block_tail_rows_match_padded_call(bmv):
    # rows < N of a ragged call equal the same rows of a call on more rows
    import torch
    say("qmv int5 tail vs padded")
    c = workloads.sb_case("int5", K=512, N=64, B=2, key="tail")
    d = case_to_dev(c)
    full = bmv.qmv_fp_block(d["x"], d["w"], d["scales"], "int5")
    part = bmv.qmv_fp_block(d["x"], d["w"][:37], d["scales"][:37], "int5")
    torch.cuda.synchronize()
    assert torch.equal(full[:, :37].contiguous().view(torch.int16), part.view(torch.int16))
