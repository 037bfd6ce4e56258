"""The entry point that allocates nothing (qmv_qvm_noalloc): called through
the C ABI, it must give the same bits as qmv_qvm with a caller workspace, on
two calls in a row, the second smaller than the first (the library's device
scratch keeps the first call's partials, which the second must not read)."""

import pytest

import workloads
from gpu_util import case_to_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bmv():
    import torch
    import bit_matrix_vector_amd as m
    assert torch.cuda.is_available()
    m.load()
    return m


def _weights(bmv, c, d):
    blk = {"affine": c.group, "mxfp4": 32, "nvfp4": 16, "mxfp8": 32}[c.fmt]
    return bmv.make_weights(c.fmt, d["w"], d["scales"], d.get("biases"), K=c.K, bits=c.bits,
                            group_size=blk, global_scale=d.get("gscale"))


def _x(c, B, key):
    rng = workloads.rng_for(11, key)
    return to_dev(workloads.to_storage(rng.normal(size=(B, c.N)), c.dtype), c.dtype)


def _pair(bmv, c, B, key):
    import torch
    d = case_to_dev(c)
    wt = _weights(bmv, c, d)
    x = _x(c, B, key)
    y_ref = bmv.qmv_qvm(x, wt)
    y = torch.full((B, c.K), float("nan"), dtype=x.dtype, device=x.device)
    bmv.qmv_qvm_noalloc(x, wt, y)
    torch.cuda.synchronize()
    return y_ref, y


def test_noalloc_qvm_two_calls_second_smaller(bmv):
    import torch
    # first: MXFP4 K=4096 N=14336 B=2 (a large split workspace); second:
    # affine 4-bit K=1024 N=300 B=1 and an f32 NVFP4 case, smaller still
    big = workloads.mlp_up_case("mxfp4", 2)
    say("noalloc qvm 1: mxfp4 bf16 B=2 K=4096 N=14336")
    a_ref, a = _pair(bmv, big, 2, "big")
    assert torch.equal(a.view(torch.int16), a_ref.view(torch.int16))
    small = workloads.affine_case(11, "noalloc-small", bits=4, group=64, K=1024, N=300, B=1,
                                  dtype="bf16")
    say("noalloc qvm 2: affine 4-bit bf16 B=1 K=1024 N=300")
    b_ref, b = _pair(bmv, small, 1, "small")
    assert torch.equal(b.view(torch.int16), b_ref.view(torch.int16))
    tiny = workloads.nvfp4_case(11, "noalloc-tiny", K=256, N=70, B=3, dtype="f32")
    say("noalloc qvm 3: nvfp4 f32 B=3 K=256 N=70")
    c_ref, c = _pair(bmv, tiny, 3, "tiny")
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))
