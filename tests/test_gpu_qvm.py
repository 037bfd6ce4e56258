"""GPU parity of qvm (y = x . W over the packed [N, K] layout) against the
oracle, with the QMV parity bar (A = sum_n |x[n] W[n, k]|)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import case_to_dev, check, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _case(fmt, bits, group, K, N, dtype, key):
    if fmt == "affine":
        return workloads.affine_case(8, key, bits=bits, group=group, K=K, N=N, B=1, dtype=dtype)
    if fmt == "mxfp4":
        return workloads.mxfp4_case(8, key, K=K, N=N, B=1, dtype=dtype)
    if fmt == "nvfp4":
        return workloads.nvfp4_case(8, key, K=K, N=N, B=1, dtype=dtype)
    return workloads.mxfp8_case(8, key, K=K, N=N, B=1, dtype=dtype)


def _run(bmv, c, B, dtype, key):
    d = case_to_dev(c)
    blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
    wt = bmv.make_weights(c.fmt, d["w"], d["scales"], d.get("biases"), K=c.K, bits=c.bits,
                          group_size=blk, global_scale=d.get("gscale"))
    x = workloads.to_storage(workloads.rng_for(8, f"qvm-x-{key}").normal(size=(B, c.N)), dtype)
    y = bmv.qmv_qvm(to_dev(x, dtype), wt)
    W = oracle.dequant(c.fmt, c.K, c.w, c.scales, c.biases, bits=c.bits, group=c.group,
                       dtype=dtype, global_scale=c.global_scale)
    return y, oracle.qvm(x, dtype, W), oracle.qvm_abs(x, dtype, W), (wt, d, x)


CASES = ([("affine", b, g) for b in (2, 3, 4, 5, 6, 8) for g in (32, 128)] +
         [("affine", 4, 64), ("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)])


@pytest.mark.parametrize("fmt,bits,group", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qvm(bmv, fmt, bits, group, dtype):
    K = {32: 1056, 64: 1088, 128: 1152, 16: 1056}[group]   # ragged column tiles
    for B in (1, 3):
        key = f"{fmt}-{bits}-{group}-{dtype}-{B}"
        say(f"qvm {key} N=300 K={K}")
        c = _case(fmt, bits, group, K, 300, dtype, key)
        y, y64, A, _ = _run(bmv, c, B, dtype, key)
        check(to_host(y, dtype), y64, A, dtype, f"qvm {key}")


@pytest.mark.parametrize("fmt,bits,group", [("affine", 4, 64), ("mxfp4", 4, 32)])
def test_qvm_f16_b8(bmv, fmt, bits, group):
    key = f"{fmt}-f16-b8"
    say(f"qvm {key}")
    c = _case(fmt, bits, group, 2048, 500, "f16", key)
    y, y64, A, _ = _run(bmv, c, 8, "f16", key)
    check(to_host(y, "f16"), y64, A, "f16", f"qvm {key}")


def test_qvm_full_size_and_repeatable(bmv):
    import torch
    say("qvm mxfp4 bf16 N=K=4096 B=1, twice")
    c = _case("mxfp4", 4, 32, 4096, 4096, "bf16", "full")
    y, y64, A, (wt, d, x) = _run(bmv, c, 1, "bf16", "full")
    check(to_host(y, "bf16"), y64, A, "bf16", "qvm full size")
    y2 = bmv.qmv_qvm(to_dev(x, "bf16"), wt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_qvm_few_rows(bmv):
    # fewer rows than waves: most waves of a block have nothing to do
    say("qvm affine 4b g64 bf16 N=3 K=512")
    c = _case("affine", 4, 64, 512, 3, "bf16", "few")
    y, y64, A, _ = _run(bmv, c, 2, "bf16", "few")
    check(to_host(y, "bf16"), y64, A, "bf16", "qvm few rows")
