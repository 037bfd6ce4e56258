"""GPU parity of the quantize-from-float entry points against the oracle:
packed codes, scales, biases and the NVFP4 global scale must match bit for
bit (every code is an integer decision both sides take in fp32)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module")
def bmv():
    import bit_matrix_vector_amd as m
    m.load()
    return m


def _host_bytes(t):
    return t.detach().cpu().numpy()


def _check_affine(bmv, w, dtype, bits, group, rows=None):
    wd = to_dev(w, dtype)
    packed, sc, bi = bmv.qmv_quantize_affine(wd, bits, group)
    ref = w if rows is None else w[rows]
    q, s, b = oracle.quantize_affine(ref, dtype, bits, group)
    got_p = _host_bytes(packed)
    got_s = to_host(sc, dtype)
    got_b = to_host(bi, dtype)
    if rows is not None:
        got_p, got_s, got_b = got_p[rows], got_s[rows], got_b[rows]
    assert np.array_equal(got_p, oracle.pack_codes(q, bits))
    if dtype == "f32" or dtype == "f16":
        got_s, s, got_b, b = (a.view(np.uint32 if dtype == "f32" else np.uint16)
                              for a in (got_s, s, got_b, b))
    assert np.array_equal(got_s, s)
    assert np.array_equal(got_b, b)
    return packed, sc, bi


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantize_affine_bit_exact(bmv, dtype, bits, group):
    say(f"quantize affine {dtype} b{bits} g{group} N=67 K=512")
    w = workloads.quant_weights(20, f"qa-{dtype}-{bits}-{group}", 67, 512, dtype)
    _check_affine(bmv, w, dtype, bits, group)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_quantize_mx_bit_exact(bmv, dtype, fmt):
    say(f"quantize {fmt} {dtype} N=67 K=1024")
    w = workloads.quant_weights(21, f"qmx-{fmt}-{dtype}", 67, 1024, dtype)
    packed, sc = bmv.qmv_quantize_mx(to_dev(w, dtype), fmt)
    codes, byte = oracle.quantize_mx(w, dtype, "e2m1" if fmt == "mxfp4" else "e4m3")
    want = oracle.pack_codes(codes, 4) if fmt == "mxfp4" else codes
    assert np.array_equal(_host_bytes(packed), want)
    assert np.array_equal(_host_bytes(sc), byte)


@pytest.mark.parametrize("dtype", DTYPES)
def test_quantize_nvfp4_bit_exact(bmv, dtype):
    say(f"quantize nvfp4 {dtype} N=67 K=1024")
    w = workloads.quant_weights(22, f"qnv-{dtype}", 67, 1024, dtype)
    packed, sc, gs = bmv.qmv_quantize_nvfp4(to_dev(w, dtype))
    codes, byte, g = oracle.quantize_nvfp4(w, dtype)
    assert np.array_equal(_host_bytes(packed), oracle.pack_codes(codes, 4))
    assert np.array_equal(_host_bytes(sc), byte)
    assert _host_bytes(gs).view(np.uint32)[0] == np.float32(g).view(np.uint32)


def test_quantize_nvfp4_repeat_call_restarts_reduction(bmv):
    # the global-scale word is the reduction's working word: a second call on
    # a smaller matrix must not see the first call's maximum
    say("quantize nvfp4 twice, second input smaller")
    w1 = workloads.quant_weights(23, "qnv-a", 16, 256, "bf16", special_rows=False)
    w2 = (workloads.quant_weights(23, "qnv-b", 16, 256, "f32", special_rows=False) * 0.01)
    w2 = w2.astype(np.float32)
    bmv.qmv_quantize_nvfp4(to_dev(w1, "bf16"))
    packed, sc, gs = bmv.qmv_quantize_nvfp4(to_dev(w2, "f32"))
    codes, byte, g = oracle.quantize_nvfp4(w2, "f32")
    assert _host_bytes(gs)[0] == g
    assert np.array_equal(_host_bytes(sc), byte)
    assert np.array_equal(_host_bytes(packed), oracle.pack_codes(codes, 4))


def test_quantize_zero_matrix_nvfp4(bmv):
    say("quantize nvfp4 all zeros")
    w = np.zeros((8, 64), np.float32)
    packed, sc, gs = bmv.qmv_quantize_nvfp4(to_dev(w, "f32"))
    assert not _host_bytes(packed).any() and not _host_bytes(sc).any()
    assert _host_bytes(gs)[0] == 0.0


@pytest.mark.parametrize("fmt", ["affine4", "mxfp4", "mxfp8", "nvfp4"])
def test_quantize_full_size_sampled_rows(bmv, fmt):
    # the bench's quantize workload (bf16 [14336, 4096]) at full size, checked
    # on sampled rows (NVFP4: the sample holds the row of the matrix maximum,
    # which fixes the global scale)
    import torch
    N, K = 14336, 4096
    say(f"quantize {fmt} bf16 N={N} K={K} sampled rows")
    w = workloads.quant_weights(24, "q-full", N, K, "bf16")
    wd = to_dev(w, "bf16")
    rows = np.unique(np.concatenate([np.arange(0, N, 997), [N - 1]]))
    if fmt == "affine4":
        _check_affine(bmv, w, "bf16", 4, 64, rows=rows)
        return
    if fmt == "nvfp4":
        wabs = np.abs(oracle.storage_to_f64(w, "bf16"))
        top = int(np.unravel_index(np.argmax(wabs), wabs.shape)[0])
        rows = np.unique(np.concatenate([rows, [top]]))
        packed, sc, gs = bmv.qmv_quantize_nvfp4(wd)
        codes, byte, g = oracle.quantize_nvfp4(w[rows], "bf16")
        assert _host_bytes(gs)[0] == g
        assert np.array_equal(_host_bytes(sc)[rows], byte)
        assert np.array_equal(_host_bytes(packed)[rows], oracle.pack_codes(codes, 4))
        return
    packed, sc = bmv.qmv_quantize_mx(wd, fmt)
    torch.cuda.synchronize()
    codes, byte = oracle.quantize_mx(w[rows], "bf16", "e2m1" if fmt == "mxfp4" else "e4m3")
    want = oracle.pack_codes(codes, 4) if fmt == "mxfp4" else codes
    assert np.array_equal(_host_bytes(packed)[rows], want)
    assert np.array_equal(_host_bytes(sc)[rows], byte)


def test_quantize_then_qmv_matches_oracle(bmv):
    # encoder output feeds the product unchanged: QMV on the device-quantized
    # MXFP4 weights equals the oracle product over the oracle-dequantized codes
    import torch
    say("quantize mxfp4 then qmv, bf16 N=300 K=2048")
    w = workloads.quant_weights(25, "q-then-qmv", 300, 2048, "bf16")
    x = workloads.to_storage(np.random.default_rng(1).normal(size=(2, 2048)), "bf16")
    packed, sc = bmv.qmv_quantize_mx(to_dev(w, "bf16"), "mxfp4")
    y = bmv.qmv_fp_mxfp4(to_dev(x, "bf16"), packed, sc)
    torch.cuda.synchronize()
    W64 = oracle.dequant("mxfp4", 2048, _host_bytes(packed), _host_bytes(sc))
    want = oracle.qmv(x, "bf16", W64)
    got = oracle.storage_to_f64(to_host(y, "bf16"), "bf16")
    ref = oracle.storage_to_f64(oracle.round_f64_to(want, "bf16"), "bf16")
    ulp = oracle.ulp_of(oracle.round_f64_to(want, "bf16"), "bf16")
    assert (np.abs(got - ref) <= ulp).all()


def test_quantize_empty_is_noop(bmv):
    import torch
    w = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    packed, sc = bmv.qmv_quantize_mx(w, "mxfp4")
    assert packed.numel() == 0 and sc.numel() == 0
