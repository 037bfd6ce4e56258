"""Pins of the Track-1 block-format oracle: E5M2 against torch's float8_e5m2
and the page's constants, two's-complement integers against NumPy's int8
arithmetic, and cross-format identities that reduce a format to one pinned
elsewhere (fp4 with power-of-two FP32 scales is MXFP4; fp8_e4m3 likewise is
MXFP8; mxint8 is int8 with the scale times 2^-6)."""

import numpy as np
import pytest
import torch

import oracle


def test_e5m2_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = oracle.e5m2_value(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(got)
    assert np.array_equal(got[ok], want[ok])


def test_e5m2_page_constants():
    # two mantissa bits, smallest normal exponent -14, largest value 57344
    assert oracle.e5m2_value(0x7B) == 57344.0
    assert oracle.e5m2_value(0x04) == 2.0 ** -14
    assert oracle.e5m2_value(0x01) == 2.0 ** -16          # smallest subnormal
    assert oracle.e5m2_value(0x3D) == 1.25                # 2^0 * (1 + 1/4)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_int_codes_two_complement(bits):
    c = np.arange(1 << bits, dtype=np.int64)
    # sign-extend through int8: shift the code to the top of a byte, then an
    # arithmetic shift back down
    want = ((c << (8 - bits)).astype(np.uint8).view(np.int8).astype(np.int64) >> (8 - bits))
    assert np.array_equal(oracle.int_value(c, bits), want.astype(np.float64))
    assert oracle.int_value((1 << bits) - 1, bits) == -1
    assert oracle.int_value(1 << (bits - 1), bits) == -(1 << (bits - 1))


def test_format_table_is_the_audit_matrix():
    f = oracle.BLOCK_FORMATS
    assert len(f) == 27                 # 30 minus mxfp4 / nvfp4 / mxfp8_e4m3
    assert f["nvfp8"] == ("e4m3", 16, "f32") and f["mxint8"] == ("int8", 32, "e8m0")
    assert f["int4"] == ("int4", 64, "f32") and f["int4_f16"] == ("int4", 64, "f16")
    assert all(b in (16, 32, 64) for _, b, _ in f.values())


def _packed(rng, N, K, bits):
    return oracle.pack_codes(rng.integers(0, 1 << bits, size=(N, K)).astype(np.uint8), bits)


def test_fp4_with_power_of_two_scales_is_mxfp4():
    rng = np.random.default_rng(0)
    N, K = 4, 128
    w = _packed(rng, N, K, 4)
    e = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    s32 = np.ldexp(1.0, e.astype(np.int32) - 127).astype(np.float32)
    assert np.array_equal(oracle.dequant("fp4", K, w, s32), oracle.dequant("mxfp4", K, w, e))
    s16 = np.ldexp(1.0, rng.integers(-10, 10, size=(N, K // 32))).astype(np.float16)
    e16 = (np.log2(s16.astype(np.float64)) + 127).astype(np.uint8)
    assert np.array_equal(oracle.dequant("fp4_f16", K, w, s16), oracle.dequant("mxfp4", K, w, e16))


def test_fp8_e4m3_with_power_of_two_scales_is_mxfp8():
    rng = np.random.default_rng(1)
    N, K = 3, 96
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0           # finite codes only
    e = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    s32 = np.ldexp(1.0, e.astype(np.int32) - 127).astype(np.float32)
    assert np.array_equal(oracle.dequant("fp8_e4m3", K, w, s32),
                          oracle.dequant("mxfp8", K, w, e))


def test_mxint8_is_int8_with_scale_times_2_pow_minus_6():
    rng = np.random.default_rng(2)
    N, K = 3, 128
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    e = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    # int8 uses blocks of 64: give both 32-blocks of a 64-block the same exponent
    e[:, 1::2] = e[:, 0::2]
    s = np.ldexp(1.0, e[:, 0::2].astype(np.int32) - 127 - 6).astype(np.float32)
    assert np.array_equal(oracle.dequant("mxint8", K, w, e), oracle.dequant("int8", K, w, s))
    # and an mxint8 code is a fixed-point number in [-2, 2)
    vals = oracle.dequant("mxint8", 32, np.arange(256, dtype=np.uint8)[None, :32],
                          np.array([[127]], np.uint8))
    assert vals.min() >= -2.0 and vals.max() < 2.0


def test_nvfp8_brute_force():
    rng = np.random.default_rng(3)
    N, K = 2, 64
    w = rng.integers(0, 127, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.01, 1.0, size=(N, K // 16)).astype(np.float32)
    W = oracle.dequant("nvfp8", K, w, s)
    for n in range(N):
        for k in range(K):
            assert W[n, k] == oracle.e4m3_value(w[n, k]) * float(s[n, k // 16])


def test_int3_bitstream_known_answer():
    # 3-bit codes 0..7 pack to 88 c6 fa (the affine known answer); as signed
    # int3 they read 0 1 2 3 -4 -3 -2 -1
    w = np.zeros((1, 12), np.uint8)
    w[0, :3] = [0x88, 0xC6, 0xFA]
    vals = oracle.dequant("int3", 32, w, np.ones((1, 1), np.float32))
    assert vals[0, :8].tolist() == [0, 1, 2, 3, -4, -3, -2, -1]
