"""Pins of the oracle's quantize-from-float encoders to facts outside
themselves: hand-worked known answers, exact recovery of matrices built from
representable values, round-half-even at every midpoint of the element grids,
saturation, and error bounds that follow from the definitions."""

import numpy as np
import pytest

import oracle
from workloads import to_storage

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f64(stored, dtype):
    return oracle.storage_to_f64(stored, dtype)


# ---- element encoders ------------------------------------------------------

def test_e2m1_encode_inverts_decode():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_encode_nearest(oracle.e2m1_value(codes)), codes)


def test_e2m1_midpoints_round_half_even():
    # magnitudes 0 .5 1 1.5 2 3 4 6 are codes 0..7; at each midpoint the even code wins
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.e2m1_encode_nearest(mids)) == want
    assert list(oracle.e2m1_encode_nearest(-np.array(mids))) == [c | 8 for c in want]
    # just above a midpoint goes up, just below goes down
    up = np.nextafter(np.array(mids), np.inf)
    dn = np.nextafter(np.array(mids), -np.inf)
    assert list(oracle.e2m1_encode_nearest(up)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(oracle.e2m1_encode_nearest(dn)) == [0, 1, 2, 3, 4, 5, 6]


def test_e2m1_saturates_and_keeps_sign_of_zero():
    assert list(oracle.e2m1_encode_nearest([6.0, 6.5, 1e30, -1e30])) == [7, 7, 7, 15]
    assert list(oracle.e2m1_encode_nearest([0.0, -0.0, -0.1])) == [0, 8, 8]


def test_e4m3_encode_inverts_decode_on_finite_bytes():
    b = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode_nearest(oracle.e4m3_value(b)), b)


def test_floor_log2_exact_over_fp32_range():
    for k in range(-149, 128):
        v = np.float32(np.ldexp(1.0, k))
        assert oracle.floor_log2(v) == k
        if k < 127:
            assert oracle.floor_log2(np.nextafter(np.float32(2.0) * v, np.float32(0))) == k


# ---- affine ------------------------------------------------------------------

def test_affine_known_answer_with_tie():
    # lo = -1, hi = 2, 2 bits -> s = 3/3 = 1, bias = -1; (0.5 + 1)/1 = 1.5 ties to 2
    w = np.array([[-1.0, 0.0, 0.5, 2.0] * 8], dtype=np.float32)
    q, s, b = oracle.quantize_affine(w, "f32", 2, 32)
    assert q.tolist() == [[0, 1, 2, 3] * 8]
    assert s.tolist() == [[1.0]] and b.tolist() == [[-1.0]]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_affine_recovers_representable_matrices(dtype, bits, group):
    # w = bias + s*q with s a power of two, bias a multiple of s, and every group
    # holding both 0 and 2^bits - 1: min and max give back s and bias exactly,
    # and every (w - bias)/s is an exact integer
    rng = np.random.default_rng(bits * 1000 + group)
    N, K = 3, 2 * group
    n = 2 ** bits - 1
    q = rng.integers(0, n + 1, size=(N, K // group, group))
    q[:, :, 0] = 0
    q[:, :, 1] = n
    s = np.ldexp(1.0, rng.integers(-9, -3, size=(N, K // group, 1)))
    # bf16 keeps 8 significant bits: 8-bit codes leave no room for a bias
    span = 0 if (dtype == "bf16" and bits == 8) else 40
    bias = s * rng.integers(-span, span + 1, size=(N, K // group, 1))
    w = (bias + s * q).reshape(N, K)
    ws = to_storage(w, dtype)
    assert np.array_equal(_f64(ws, dtype), w)          # representable in T
    qq, ss, bb = oracle.quantize_affine(ws, dtype, bits, group)
    assert np.array_equal(qq, q.reshape(N, K))
    assert np.array_equal(_f64(ss, dtype), s[:, :, 0])
    assert np.array_equal(_f64(bb, dtype), bias[:, :, 0])


def test_affine_constant_group_is_bias_only():
    w = np.full((2, 64), 0.3, dtype=np.float32)
    q, s, b = oracle.quantize_affine(w, "f32", 4, 64)
    assert not q.any() and not s.any()
    assert np.array_equal(b, np.full((2, 1), np.float32(0.3)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_affine_error_bound(dtype, bits):
    # every element lands within half a step of its value, plus what storing s
    # and bias in T moved them (a clamped top code is off by n*|s32 - s|)
    rng = np.random.default_rng(bits)
    w = to_storage(rng.normal(0, 1, size=(16, 256)), dtype)
    q, s, b = oracle.quantize_affine(w, dtype, bits, 64)
    w64 = _f64(w, dtype)
    g = w64.reshape(16, 4, 64)
    lo, hi = g.min(axis=2), g.max(axis=2)
    s32 = ((hi.astype(np.float32) - lo.astype(np.float32)) / np.float32(2 ** bits - 1))
    sd, bd = _f64(s, dtype), _f64(b, dtype)
    deq = oracle.dequant_affine(oracle.pack_codes(q, bits), s, b, 256, bits, 64, dtype)
    err = np.abs(deq - w64).reshape(16, 4, 64).max(axis=2)
    bound = (sd / 2 + (2 ** bits - 1) * np.abs(s32 - sd) + np.abs(lo - bd)) * (1 + 1e-6) + 1e-30
    assert (err <= bound).all()


# ---- MX ------------------------------------------------------------------------

def test_mx_known_answers_e2m1():
    # amax 6 -> floor(log2 6) - 2 = 0 -> byte 127; amax 7 -> same byte, 7 saturates;
    # amax 8 -> byte 128, X = 2, 8/2 = 4 (code 6)
    base = np.zeros((3, 32), dtype=np.float32)
    base[0, :4] = [6, -3, 0.5, 0.25]
    base[1, :2] = [7, 1.0]
    base[2, :2] = [8, -1.0]
    codes, byte = oracle.quantize_mx(base, "f32", "e2m1")
    assert byte[:, 0].tolist() == [127, 127, 128]
    assert codes[0, :4].tolist() == [7, 13, 1, 0]
    assert codes[1, :2].tolist() == [7, 2]
    assert codes[2, :2].tolist() == [6, 9]
    assert codes[:, 4:].max() == 0


def test_mx_known_answers_e4m3():
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, :3] = [448.0, -1.0, 2.0 ** -9]        # floor(log2 448) - 8 = 0 -> byte 127
    w[1, 0] = 1.0                              # -8 -> byte 119, 1/2^-8 = 256 -> 0x78
    codes, byte = oracle.quantize_mx(w, "f32", "e4m3")
    assert byte[:, 0].tolist() == [127, 119]
    assert codes[0, :3].tolist() == [0x7E, 0xB8, 0x01]
    assert codes[1, 0] == 0x78


def test_mx_zero_block_and_byte_clamp():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 32] = np.float32(2.0 ** -149)         # log2 = -149 -> clamps to byte 0
    codes, byte = oracle.quantize_mx(w, "f32", "e2m1")
    assert byte.tolist() == [[0, 0]]
    assert not codes[0, :32].any()
    # 2^-149 / 2^-127 = 2^-22 rounds to 0
    assert codes[0, 32] == 0


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_recovers_representable_blocks(elem):
    # blocks of element values times 2^k whose largest magnitude is the format's
    # largest value: the chosen exponent is k and dequantization is exact
    rng = np.random.default_rng(3)
    top = 6.0 if elem == "e2m1" else 448.0
    vals = oracle.e2m1_value(np.arange(16)) if elem == "e2m1" else \
        oracle.e4m3_value(np.array([c for c in range(256) if c & 0x7F != 0x7F]))
    N, K = 4, 128
    el = rng.choice(vals, size=(N, K // 32, 32))
    el[:, :, 0] = top
    k = rng.integers(-20, 20, size=(N, K // 32, 1))
    w = (el * np.ldexp(1.0, k)).reshape(N, K).astype(np.float32)
    codes, byte = oracle.quantize_mx(w, "f32", elem)
    assert np.array_equal(byte.astype(np.int64), k[:, :, 0] + 127)
    dec = oracle.e2m1_value(codes) if elem == "e2m1" else oracle.e4m3_value(codes)
    deq = dec.reshape(N, K // 32, 32) * oracle.e8m0_value(byte)[:, :, None]
    assert np.array_equal(deq.reshape(N, K), w.astype(np.float64))


def test_mx_elements_are_nearest_to_scaled_value():
    # brute force on one block: each code's value is a nearest grid point of w/X
    rng = np.random.default_rng(4)
    w = rng.normal(0, 1, size=(1, 32)).astype(np.float32)
    codes, byte = oracle.quantize_mx(w, "f32", "e2m1")
    X = 2.0 ** (int(byte[0, 0]) - 127)
    t = w[0].astype(np.float64) / X
    grid = oracle.e2m1_value(np.arange(16))
    for tj, c in zip(t, codes[0]):
        d = np.abs(grid - np.clip(tj, -6, 6))
        assert abs(oracle.e2m1_value(c) - np.clip(tj, -6, 6)) == d.min()


# ---- NVFP4 ---------------------------------------------------------------------

def test_nvfp4_two_levels_known_answer():
    # A = 2688 -> global 1; block 0 holds A: 2688/6/1 = 448 -> 0x7E; block 1 max
    # 3 -> 0.5 -> E4M3 0x30; its elements are w / 0.5
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 2688.0
    w[0, 1] = -448.0
    w[0, 16:19] = [3.0, -1.5, 0.25]
    codes, byte, gs = oracle.quantize_nvfp4(w, "f32")
    assert gs == np.float32(1.0)
    assert byte.tolist() == [[0x7E, 0x30]]
    assert codes[0, :2].tolist() == [7, 10]         # 6 and -1
    assert codes[0, 16:19].tolist() == [7, 13, 1]   # 6, -3, 0.5


def test_nvfp4_all_zero():
    codes, byte, gs = oracle.quantize_nvfp4(np.zeros((2, 32), np.float32), "f32")
    assert gs == 0 and not codes.any() and not byte.any()


def test_nvfp4_error_bound():
    # within half an element step after the scale rounding, or saturated at 6
    rng = np.random.default_rng(5)
    w = rng.normal(0, 1, size=(8, 64)).astype(np.float32)
    codes, byte, gs = oracle.quantize_nvfp4(w, "f32")
    d = oracle.e4m3_value(byte).astype(np.float64) * float(gs)
    deq = oracle.e2m1_value(codes).reshape(8, 4, 16) * d[:, :, None]
    t = w.reshape(8, 4, 16) / d[:, :, None]
    err = np.abs(deq - w.reshape(8, 4, 16))
    step = np.where(np.abs(t) < 2, 0.5, np.where(np.abs(t) < 4, 1.0, 2.0)) * d[:, :, None]
    sat = np.abs(t) > 6
    assert ((err <= step / 2 * (1 + 1e-6)) | sat).all()
