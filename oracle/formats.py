"""Element and scale decoders of the block-scaled formats, from their closed
forms, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* E2M1 (4-bit float element of MXFP4 / NVFP4): 1 sign, 2 exponent, 1 mantissa
  bit. "wh-iron kernel-op coverage audit", op-coverage table, row
  fp_quantized_nax, lists its magnitudes: {0, 0.5, 1, 1.5, 2, 3, 4, 6} plus a
  sign bit.
* E4M3 (8-bit float element of MXFP8, block scale of NVFP4), OCP "fn" variant:
  1 sign, 4 exponent, 3 mantissa bits, exponent bias 7. The same audit's
  kv_cache row gives mantissa_bits = 3, smallest normal exponent -6 and max
  448; its "Model-format decode" table keeps the NaN sentinel explicit. In the
  fn variant there is no infinity and S.1111.111 is the only NaN pattern.
* E8M0 (MX block scale): an unsigned biased exponent, value 2^(e-127), with
  0xFF reserved for NaN (OCP MX; the audit's format table calls it a pow-2
  scale of one byte).
"""

from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """fp64 value of E2M1 codes (uint8, low 4 bits used).

    sign = bit 3, exponent field e = bits 2..1, mantissa m = bit 0;
    e == 0: 0.5*m (zero or the subnormal 0.5), else 2^(e-1) * (1 + m/2)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32)))
    return sign * mag


def e4m3_value(byte) -> np.ndarray:
    """fp64 value of OCP E4M3 (e4m3fn) bytes.

    sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: subnormal m * 2^-9; e == 15 and m == 7: NaN; else
    2^(e-7) * (1 + m/8). Largest finite value 448 (0x7E)."""
    b = np.asarray(byte, dtype=np.int64) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9,
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    val = sign * mag
    return np.where((e == 15) & ((b & 7) == 7), np.nan, val)


def e8m0_value(byte) -> np.ndarray:
    """fp64 value of E8M0 bytes: 2^(e-127) for e in 0..254, NaN for 255.
    (e = 0 is 2^-127, a subnormal in fp32 but normal in fp64.)"""
    b = np.asarray(byte, dtype=np.int64) & 0xFF
    return np.where(b == 255, np.nan, np.ldexp(1.0, (b - 127).astype(np.int32)))


_E4M3_POS_CODES = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E finite
_E4M3_POS_VALUES = e4m3_value(_E4M3_POS_CODES)               # increasing


def nearest_code(a, values) -> np.ndarray:
    """Index of the entry of the increasing array `values` nearest to each
    a >= 0 (a no larger than values[-1]); an exact tie between two entries goes
    to the even index. With values listed in code order this is the nearest
    code, ties to the code whose lowest bit is 0."""
    a = np.asarray(a, dtype=np.float64)
    idx = np.searchsorted(values, a)                 # first entry >= a
    hi = np.clip(idx, 0, len(values) - 1)
    lo = np.clip(idx - 1, 0, len(values) - 1)
    dlo = a - values[lo]
    dhi = values[hi] - a
    tie = np.where(lo % 2 == 0, lo, hi)
    return np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, tie))


def e4m3_encode_nearest(v) -> np.ndarray:
    """Reference for the E4M3 encoders: the E4M3 byte nearest to v.

    Defined by search over the 127 non-negative finite values, not by bit
    manipulation: the nearest value wins; an exact tie goes to the even code
    (the code whose mantissa LSB is 0, i.e. round-half-to-even); magnitudes
    above 448 saturate to 448 (0x7E); the sign goes to bit 7 (so -0.0 gives
    0x80); NaN gives 0x7F. Infinities saturate like any large value."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(np.nan_to_num(v, nan=0.0)), 448.0)
    code = nearest_code(a, _E4M3_POS_VALUES).astype(np.uint8)
    code = np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)
