"""C-ABI tests that need no GPU: the library loads, exports every function
include/qmv.h declares, rejects bad arguments before any HIP call, and its
host codecs agree byte for byte with the oracle."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import bit_matrix_vector_amd as bmv

V = ctypes.c_void_p
OK, INVAL, UNSUP, MISAL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return bmv.load()


def test_library_exports_every_header_function(lib):
    names = bmv.header_functions()
    assert {"qmv_affine", "qmv_fp_mxfp4", "qmv_fp_nvfp4", "qmv_fp_mxfp8", "gather_qmv",
            "qmv_pack_codes", "qmv_unpack_codes", "qmv_encode_e4m3",
            "qmv_unpack_codes_device", "qmv_dequant_device", "qmv_packed_row_bytes",
            "qmv_quantize_affine", "qmv_quantize_mxfp4", "qmv_quantize_mxfp8",
            "qmv_quantize_nvfp4", "qmv_moe_gate_up_swiglu", "qmv_moe_down_reduce", "qmv_fp_block",
            "qmv_qvm", "qmv_qvm_workspace_bytes", "qmv_qmm", "qmv_qmm_workspace_bytes",
            "qmv_qvm_noalloc", "qmv_qvm_noalloc_max_workspace_bytes",
            "qmv_rmsnorm_qmv", "gather_qmm",
            "qmv_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


# fake, suitably aligned device addresses: validation must reject before use
X, W, S, Bi, Y = V(0x10000), V(0x20000), V(0x30000), V(0x40000), V(0x50000)


def _affine(lib, **kw):
    a = dict(stream=None, dtype=2, B=1, K=64, N=8, x=X, w=W, s=S, b=Bi, bits=4, group=64, y=Y)
    a.update(kw)
    return lib.qmv_affine(a["stream"], a["dtype"], a["B"], a["K"], a["N"], a["x"], a["w"],
                          a["s"], a["b"], a["bits"], a["group"], a["y"])


@pytest.mark.parametrize("kw,status,word", [
    (dict(dtype=7), INVAL, "dtype"),
    (dict(bits=7), UNSUP, "bits"),
    (dict(bits=1), UNSUP, "bits"),
    (dict(group=16), UNSUP, "group"),
    (dict(K=48), INVAL, "multiple of 32"),
    (dict(K=96, group=64), INVAL, "group"),
    (dict(B=9), UNSUP, "batch"),
    (dict(K=(1 << 24) + 64), UNSUP, "2^24"),
    (dict(N=(1 << 28) + 1), UNSUP, "2^28"),
    (dict(B=-1), INVAL, "negative"),
    (dict(N=-2), INVAL, "negative"),
    (dict(x=None), INVAL, "x is NULL"),
    (dict(w=None), INVAL, "w is NULL"),
    (dict(s=None), INVAL, "scales is NULL"),
    (dict(y=None), INVAL, "y is NULL"),
    (dict(x=V(0x10008)), MISAL, "x is not 16-byte"),
    (dict(w=V(0x20004)), MISAL, "w is not 16-byte"),
    (dict(y=V(0x50001)), MISAL, "y is not 2-byte"),
    (dict(dtype=0, s=V(0x30002)), MISAL, "scales is not 4-byte"),
    (dict(x=V(0x50000)), INVAL, "overlap"),
])
def test_affine_validation(lib, kw, status, word):
    assert _affine(lib, **kw) == status
    assert word in lib.qmv_last_error().decode()


def test_empty_calls_are_noops(lib):
    assert _affine(lib, B=0, x=None, w=None, s=None, b=None, y=None) == OK
    assert _affine(lib, N=0, x=None, w=None, s=None, b=None, y=None) == OK
    assert lib.qmv_fp_mxfp4(None, 2, 0, 4096, 16, None, None, None, None) == OK


def test_fp_validation(lib):
    assert lib.qmv_fp_mxfp4(None, 2, 1, 4096, 16, X, W, S, None) == INVAL
    assert lib.qmv_fp_nvfp4(None, 2, 1, 4096, 16, X, W, V(0x30001), None, Y) == MISAL
    assert "scales" in lib.qmv_last_error().decode()
    assert lib.qmv_fp_nvfp4(None, 2, 1, 4096, 16, X, W, S, V(0x60002), Y) == MISAL
    assert "global_scale" in lib.qmv_last_error().decode()
    assert lib.qmv_fp_mxfp8(None, 2, 1, 4080, 16, X, W, S, Y) == INVAL
    assert lib.qmv_fp_mxfp8(None, 2, 12, 4096, 16, X, W, S, Y) == UNSUP


def test_gather_validation(lib):
    wt = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 64, 1536, 4096, 0x20000, 0x30000, None, None)
    lhs, rhs = V(0x70000), V(0x80000)
    assert lib.gather_qmv(None, 2, None, X, 16, lhs, rhs, 128, Y) == INVAL
    assert lib.gather_qmv(None, 2, ctypes.byref(wt), X, 16, None, rhs, 128, Y) == INVAL
    assert lib.gather_qmv(None, 2, ctypes.byref(wt), X, 16, lhs, V(0x80002), 128, Y) == MISAL
    assert lib.gather_qmv(None, 2, ctypes.byref(wt), X, 16, lhs, rhs, 0, None) == OK
    bad = bmv.QmvWeights(bmv.QMV_AFFINE, 7, 64, 4, 16, 4096, 0x20000, 0x30000, 0x40000, None)
    assert lib.gather_qmv(None, 2, ctypes.byref(bad), X, 16, lhs, rhs, 8, Y) == UNSUP
    neg = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, -1, 16, 4096, 0x20000, 0x30000, None, None)
    assert lib.gather_qmv(None, 2, ctypes.byref(neg), X, 16, lhs, rhs, 8, Y) == INVAL


def test_device_codec_validation(lib):
    assert lib.qmv_unpack_codes_device(None, W, 4, 48, 4, V(0x90000)) == INVAL
    assert lib.qmv_unpack_codes_device(None, W, 4, 64, 7, V(0x90000)) == UNSUP
    wt = bmv.QmvWeights(bmv.QMV_MXFP8, 8, 32, 2, 16, 64, 0x20000, 0x30000, None, None)
    assert lib.qmv_dequant_device(None, 2, ctypes.byref(wt), V(0x90000)) == INVAL


def test_qvm_validation(lib):
    ws = V(0xA0000)
    wt = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 1, 300, 1024, 0x20000, 0x30000, None, None)
    need = lib.qmv_qvm_workspace_bytes(2, 1024, 300)
    assert need > 0 and need % 4 == 0
    assert lib.qmv_qvm(None, 2, ctypes.byref(wt), 2, X, Y, ws, need - 4) == INVAL
    assert "workspace" in lib.qmv_last_error().decode()
    assert lib.qmv_qvm(None, 2, ctypes.byref(wt), 9, X, Y, ws, need) == UNSUP
    assert lib.qmv_qvm(None, 2, ctypes.byref(wt), 2, X, Y, None, need) == INVAL
    assert lib.qmv_qvm(None, 2, ctypes.byref(wt), 2, X, V(0x10000), ws, need) == INVAL  # overlap
    two = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 2, 300, 1024, 0x20000, 0x30000, None, None)
    assert lib.qmv_qvm(None, 2, ctypes.byref(two), 2, X, Y, ws, need) == INVAL
    sb = bmv.QmvWeights(5, 14, 64, 1, 300, 1024, 0x20000, 0x30000, None, None)
    assert lib.qmv_qvm(None, 2, ctypes.byref(sb), 2, X, Y, ws, need) == UNSUP
    assert lib.qmv_qvm(None, 2, ctypes.byref(wt), 0, X, Y, None, 0) == OK


def test_qvm_noalloc_validation(lib):
    # the entry point without a workspace: same checks as qmv_qvm, plus the
    # library scratch's limit, all before any HIP call
    lim = lib.qmv_qvm_noalloc_max_workspace_bytes()
    assert lim == 16 << 20
    wt = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 1, 300, 1024, 0x20000, 0x30000, None, None)
    assert lib.qmv_qvm_noalloc(None, 2, ctypes.byref(wt), 9, X, Y) == UNSUP
    assert lib.qmv_qvm_noalloc(None, 2, ctypes.byref(wt), 2, None, Y) == INVAL
    assert lib.qmv_qvm_noalloc(None, 2, ctypes.byref(wt), 2, X, V(0x10000)) == INVAL
    assert lib.qmv_qvm_noalloc(None, 2, ctypes.byref(wt), 0, X, Y) == OK
    # K = 16384, N = 32769 at B = 8 needs more split partials than the scratch
    big = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 1, 32769, 16384, 0x20000, 0x30000, None, None)
    assert lib.qmv_qvm_workspace_bytes(8, 16384, 32769) > lim
    assert lib.qmv_qvm_noalloc(None, 2, ctypes.byref(big), 8, X, V(0x10000000)) == UNSUP
    msg = lib.qmv_last_error().decode()
    assert "scratch" in msg and "qmv_qvm_noalloc" in msg


def test_block_format_validation(lib):
    f = lib.qmv_fp_block
    E8, F32, F16 = 4, 5, 6
    assert f(None, 2, 3, 2, 32, 1, 512, 16, X, W, S, Y) == INVAL          # not the family
    assert f(None, 2, E8, 2, 32, 1, 512, 16, X, W, S, Y) == UNSUP         # E4M3/E8M0 is mxfp8
    assert f(None, 2, E8, 1, 32, 1, 512, 16, X, W, S, Y) == UNSUP         # E2M1/E8M0 is mxfp4
    assert f(None, 2, F32, 2, 64, 1, 512, 16, X, W, S, Y) == UNSUP        # floats use 16 / 32
    assert f(None, 2, F32, 14, 32, 1, 512, 16, X, W, S, Y) == UNSUP       # ints use 64 (F32)
    assert f(None, 2, F32, 17, 64, 1, 512, 16, X, W, S, Y) == UNSUP       # int7 does not exist
    assert f(None, 2, F32, 14, 64, 1, 544, 16, X, W, S, Y) == INVAL       # K % block
    assert f(None, 2, F32, 14, 64, 1, 512, 16, X, W, V(0x30002), Y) == MISAL   # FP32 scales
    assert f(None, 2, F16, 14, 64, 1, 512, 16, X, W, V(0x30001), Y) == MISAL   # FP16 scales
    assert f(None, 2, F16, 2, 16, 1, 512, 0, X, W, S, Y) == OK            # N = 0
    wt = bmv.QmvWeights(F32, 14, 64, 4, 16, 512, 0x20000, 0x30000, None, None)
    assert lib.gather_qmv(None, 2, ctypes.byref(wt), X, 16, V(0x70000), V(0x80000), 8,
                          Y) == UNSUP


def test_moe_validation(lib):
    ids, r, M = V(0x70000), V(0x80000), V(0x90000)
    g = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 64, 1536, 4096, 0x20000, 0x30000, None, None)
    u8 = bmv.QmvWeights(bmv.QMV_MXFP8, 8, 32, 64, 1536, 4096, 0x20000, 0x30000, None, None)
    f = lib.qmv_moe_gate_up_swiglu
    assert f(None, 2, None, ctypes.byref(g), X, 16, ids, 8, 0.0, M) == INVAL
    assert f(None, 2, ctypes.byref(g), ctypes.byref(u8), X, 16, ids, 8, 0.0, M) == INVAL
    assert "differ" in lib.qmv_last_error().decode()
    assert f(None, 2, ctypes.byref(g), ctypes.byref(g), X, 16, ids, 0, 0.0, M) == INVAL
    assert f(None, 2, ctypes.byref(g), ctypes.byref(g), X, 16, None, 8, 0.0, M) == INVAL
    assert f(None, 2, ctypes.byref(g), ctypes.byref(g), V(0x10008), 16, ids, 8, 0.0, M) == MISAL
    big = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 4, 64, 32768, 0x20000, 0x30000, None, None)
    assert f(None, 2, ctypes.byref(big), ctypes.byref(big), X, 2, ids, 2, 0.0, M) == UNSUP
    assert f(None, 2, ctypes.byref(g), ctypes.byref(g), X, 0, ids, 8, 0.0, M) == OK
    d = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 64, 4096, 1536, 0x20000, 0x30000, None, None)
    h = lib.qmv_moe_down_reduce
    assert h(None, 2, ctypes.byref(d), M, 16, ids, r, 17, Y) == UNSUP
    d2 = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 64, 4096, 8192, 0x20000, 0x30000, None, None)
    assert h(None, 2, ctypes.byref(d2), M, 16, ids, r, 8, Y) == UNSUP
    assert h(None, 2, ctypes.byref(d), M, 16, ids, None, 8, Y) == INVAL
    assert h(None, 2, ctypes.byref(d), M, 16, ids, V(0x80002), 8, Y) == MISAL
    assert h(None, 2, ctypes.byref(d), M, -1, ids, r, 8, Y) == INVAL
    assert h(None, 2, ctypes.byref(d), M, 0, ids, r, 8, Y) == OK


def test_quantize_validation(lib):
    P = V(0x90000)
    qa = lib.qmv_quantize_affine
    assert qa(None, 9, 16, 512, W, 4, 64, P, S, Bi) == INVAL
    assert qa(None, 2, 16, 512, W, 7, 64, P, S, Bi) == UNSUP
    assert qa(None, 2, 16, 512, W, 4, 48, P, S, Bi) == UNSUP
    assert qa(None, 2, 16, 96, W, 4, 64, P, S, Bi) == INVAL
    assert qa(None, 2, 16, 500, W, 4, 32, P, S, Bi) == INVAL
    assert qa(None, 2, -1, 512, W, 4, 64, P, S, Bi) == INVAL
    assert qa(None, 2, 16, 512, V(0x20008), 4, 64, P, S, Bi) == MISAL
    assert "w is not 16-byte" in lib.qmv_last_error().decode()
    assert qa(None, 2, 16, 512, W, 4, 64, V(0x90004), S, Bi) == MISAL
    assert qa(None, 2, 16, 512, W, 4, 64, P, None, Bi) == INVAL
    assert qa(None, 2, 16, 512, W, 4, 64, P, S, V(0x40001)) == MISAL
    assert qa(None, 2, 0, 512, None, 4, 64, None, None, None) == OK
    assert lib.qmv_quantize_mxfp4(None, 2, 16, 48, W, P, S) == INVAL
    assert lib.qmv_quantize_mxfp8(None, 2, 16, 64, W, None, S) == INVAL
    assert lib.qmv_quantize_nvfp4(None, 2, 16, 64, W, P, S, None) == INVAL
    assert "global_scale" in lib.qmv_last_error().decode()
    assert lib.qmv_quantize_nvfp4(None, 2, 16, 64, W, P, S, V(0x60002)) == MISAL
    assert lib.qmv_quantize_nvfp4(None, 2, 16, 0, None, None, None, None) == OK


@pytest.mark.parametrize("fmt,bits,K,expect", [
    ("affine", 3, 4096, 1536), ("affine", 5, 64, 40), ("affine", 8, 32, 32),
    ("mxfp4", 4, 4096, 2048), ("nvfp4", 4, 4096, 2048), ("mxfp8", 8, 4096, 4096),
    ("affine", 7, 64, -1),
])
def test_packed_row_bytes(fmt, bits, K, expect):
    assert bmv.qmv_packed_row_bytes(fmt, bits, K) == expect
    if expect > 0 and fmt == "affine":
        assert expect == oracle.packed_row_bytes(K, bits)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_host_pack_matches_oracle_packer(bits):
    rng = np.random.default_rng(100 + bits)
    codes = rng.integers(0, 1 << bits, size=(7, 256), dtype=np.uint8)
    packed = bmv.qmv_pack_codes(codes, bits)
    assert np.array_equal(packed, oracle.pack_codes(codes, bits))
    assert np.array_equal(bmv.qmv_unpack_codes(packed, 256, bits), codes)
    assert np.array_equal(bmv.qmv_unpack_codes(packed, 256, bits),
                          oracle.unpack_codes(packed, 256, bits))


def test_host_pack_rejects_wide_codes():
    with pytest.raises(bmv.QmvError) as e:
        bmv.qmv_pack_codes(np.array([[0, 8] * 16], dtype=np.uint8), 3)
    assert "does not fit" in str(e.value)


def test_host_e4m3_encoder_matches_oracle():
    rng = np.random.default_rng(11)
    vals = oracle.e4m3_value(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2
    v = np.concatenate([
        rng.normal(0, 1, 5000), rng.normal(0, 100, 2000), rng.uniform(-2 ** -6, 2 ** -6, 2000),
        rng.uniform(-1e-4, 1e-4, 500), vals, -vals, mids, -mids,
        [0.0, -0.0, 447.9, 448.0, 449.0, 464.0, 1e9, -1e9, np.inf, -np.inf, np.nan,
         2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -11],
    ]).astype(np.float32)
    got = bmv.qmv_encode_e4m3(v)
    ref = oracle.e4m3_encode_nearest(v.astype(np.float64))
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_qvm_split_bounds(lib):
    # a split holds between 64 * B and 8192 / B rows (when N allows), so the
    # workspace stays a small fraction of the weights and x fits LDS
    for B, K, N in ((1, 4096, 14336), (8, 4096, 14336), (1, 512, 1 << 20), (3, 14336, 4096),
                    (1, 4096, 100), (8, 512, 1 << 22)):
        ws = lib.qmv_qvm_workspace_bytes(B, K, N)
        splits = ws // (B * K * 4)
        rps = -(-N // splits)
        assert rps <= 8192 // B
        assert splits <= max(-(-N // (64 * B)), -(-N // (8192 // B)))
    assert lib.qmv_qvm_workspace_bytes(1, 4096, 14336) == 112 * 4096 * 4
    assert lib.qmv_qvm_workspace_bytes(1, 4096, 4096) == 64 * 4096 * 4


def test_qmm_validation(lib):
    wt = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 1, 300, 1024, 0x20000, 0x30000, None, None)
    ws = V(0xA0000)
    need = lib.qmv_qmm_workspace_bytes(16, 1024, 300, bmv.QMV_MXFP4)
    assert need > 0 and need % (16 * 300 * 4) == 0          # few tiles: K is split
    assert lib.qmv_qmm_workspace_bytes(4096, 4096, 14336, bmv.QMV_MXFP4) == 0  # many tiles
    assert lib.qmv_qmm(None, 0, ctypes.byref(wt), 16, X, Y, ws, need) == UNSUP    # f32
    assert lib.qmv_qmm(None, 7, ctypes.byref(wt), 16, X, Y, ws, need) == INVAL    # not a dtype
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), -1, X, Y, ws, need) == INVAL
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 65535 * 64 + 1, X, Y, ws, need) == UNSUP
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 16, V(0x100008), Y, ws, need) == MISAL
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 16, X, X, ws, need) == INVAL    # overlap
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 16, X, Y, ws, need - 4) == INVAL
    assert "workspace" in lib.qmv_last_error().decode()
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 16, X, Y, None, need) == INVAL
    two = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 2, 300, 1024, 0x20000, 0x30000, None, None)
    assert lib.qmv_qmm(None, 2, ctypes.byref(two), 16, X, Y, ws, need) == INVAL
    sb = bmv.QmvWeights(5, 14, 64, 1, 300, 1024, 0x20000, 0x30000, None, None)
    assert lib.qmv_qmm(None, 2, ctypes.byref(sb), 16, X, Y, ws, need) == UNSUP
    odd = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 1, 300, 1000, 0x20000, 0x30000, None, None)
    assert lib.qmv_qmm(None, 2, ctypes.byref(odd), 16, X, Y, ws, need) == INVAL   # K % 32
    assert lib.qmv_qmm(None, 2, ctypes.byref(wt), 0, X, Y, None, 0) == OK         # M == 0
    assert lib.qmv_qmm(None, 2, None, 16, X, Y, ws, need) == INVAL


def test_qmm_split_rule(lib):
    # splits only when the output tiles (128 or 64 rows x 128 columns) are
    # fewer than 256, at most 8, each split at least 8 slices of 64 codes,
    # none empty; affine codes always take 64-row tiles
    for fmt in (bmv.QMV_MXFP4, bmv.QMV_AFFINE):
        for M, K, N in ((32, 4096, 14336), (9, 1056, 300), (256, 4096, 4096), (1, 512, 64),
                        (64, 8192, 4096), (2000, 4096, 14336), (256, 4096, 14336)):
            ws = lib.qmv_qmm_workspace_bytes(M, K, N, fmt)
            s = ws // (M * N * 4) if ws else 1
            t128 = -(-M // 128) * -(-N // 128)
            bm = 128 if M > 64 and fmt != bmv.QMV_AFFINE and t128 >= 256 else 64
            tiles = -(-N // 128) * -(-M // bm)
            nk = -(-K // 64)
            assert 1 <= s <= 8
            if tiles >= 256:
                assert s == 1
            if s > 1:
                per = -(-nk // s)
                assert per >= 8 and (s - 1) * per < nk


def test_gather_qmm_validation(lib):
    f = lib.gather_qmm
    lhs, rhs = V(0x60000), V(0x70000)
    wt = bmv.QmvWeights(bmv.QMV_MXFP4, 4, 32, 4, 300, 1024, 0x20000, 0x30000, None, None)
    assert f(None, 0, ctypes.byref(wt), X, 16, lhs, rhs, 64, Y) == UNSUP      # f32
    assert f(None, 2, ctypes.byref(wt), X, 16, lhs, rhs, -1, Y) == INVAL
    assert f(None, 2, ctypes.byref(wt), X, -1, lhs, rhs, 64, Y) == INVAL
    assert f(None, 2, ctypes.byref(wt), X, 16, lhs, rhs, 65535 * 64 + 1, Y) == UNSUP
    assert f(None, 2, ctypes.byref(wt), X, 16, None, rhs, 64, Y) == INVAL
    assert f(None, 2, ctypes.byref(wt), X, 16, lhs, V(0x70002), 64, Y) == MISAL
    assert f(None, 2, ctypes.byref(wt), X, 16, lhs, rhs, 64, X) == INVAL      # x and y overlap
    sb = bmv.QmvWeights(5, 14, 64, 4, 300, 1024, 0x20000, 0x30000, None, None)
    assert f(None, 2, ctypes.byref(sb), X, 16, lhs, rhs, 64, Y) == UNSUP
    assert f(None, 2, ctypes.byref(wt), X, 16, lhs, rhs, 0, Y) == OK          # no slots
    assert f(None, 2, None, X, 16, lhs, rhs, 64, Y) == INVAL
