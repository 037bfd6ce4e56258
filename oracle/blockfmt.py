"""Symmetric block-scaled formats beyond MXFP4 / NVFP4 / MXFP8: the rest of the
Track-1 format matrix, each an element code times a per-block scale, no zero
point.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "wh-iron kernel-op coverage audit", section "Quantization precision
coverage": formats vary along element (signed int2..int8, or the E2M1 / E4M3 /
E5M2 micro-floats), block (16 / 32 / 64 along K) and scale storage (E8M0 power
of two, FP32, or FP16 for the *_f16 twins); the Track-1 table lists the
combinations; sub-byte codes are packed LSB first (a 4-bit stream is the usual
nibble layout), 8-bit codes are bytes. Its kv_cache op row gives E5M2 as 2
mantissa bits, smallest normal exponent -14, largest value 57344 (OCP E5M2:
exponent bias 15, subnormals m * 2^-16, exponent 31 holds infinity (m = 0)
and NaN).

Readings: the integer elements are two's-complement codes of their width,
value = code * scale. For the mxint formats (E8M0 block scale) the audit says
mxint8 is OCP's MXINT8 and the other widths follow the same construction;
OCP's MXINT8 reads its int8 element as a fixed-point number with an implicit
factor 2^-6, so an n-bit mxint element is read as code * 2^-(n-2) (one sign
bit, one integer bit, n - 2 fraction bits). FP16 scales are IEEE binary16
(subnormals included).
"""

from __future__ import annotations

import numpy as np

from .codes import unpack_codes
from .formats import e2m1_value, e4m3_value, e8m0_value


def e5m2_value(byte) -> np.ndarray:
    """fp64 value of OCP E5M2 bytes: sign bit 7, exponent bits 6..2 (bias 15),
    mantissa bits 1..0; e == 0: m * 2^-16; e == 31: infinity (m == 0) or NaN;
    else 2^(e-15) * (1 + m/4)."""
    b = np.asarray(byte, dtype=np.int64) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 2) & 0x1F
    m = (b & 3).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -16, np.ldexp(1.0 + m / 4.0, (e - 15).astype(np.int32)))
    mag = np.where((e == 31) & (m == 0), np.inf, mag)
    mag = np.where((e == 31) & (m != 0), np.nan, mag)
    return sign * mag


def int_value(code, bits: int) -> np.ndarray:
    """Two's-complement value of `bits`-wide codes (the low bits of `code`)."""
    c = np.asarray(code, dtype=np.int64) & ((1 << bits) - 1)
    return np.where(c >= 1 << (bits - 1), c - (1 << bits), c).astype(np.float64)


ELEMENTS = {  # name -> code width in bits
    "e2m1": 4, "e4m3": 8, "e5m2": 8,
    "int2": 2, "int3": 3, "int4": 4, "int5": 5, "int6": 6, "int8": 8,
}

# The Track-1 formats this module covers: name -> (element, block, scale).
FORMATS = {
    "mxfp8_e5m2": ("e5m2", 32, "e8m0"),
    "nvfp8": ("e4m3", 16, "f32"),
    "fp4": ("e2m1", 32, "f32"),
    "fp8_e4m3": ("e4m3", 32, "f32"),
    "fp8_e5m2": ("e5m2", 32, "f32"),
    **{f"int{n}": (f"int{n}", 64, "f32") for n in (2, 3, 4, 5, 6, 8)},
    **{f"mxint{n}": (f"int{n}", 32, "e8m0") for n in (2, 3, 4, 5, 6, 8)},
    "nvfp8_f16": ("e4m3", 16, "f16"),
    "fp4_f16": ("e2m1", 32, "f16"),
    "fp8_e4m3_f16": ("e4m3", 32, "f16"),
    "fp8_e5m2_f16": ("e5m2", 32, "f16"),
    **{f"int{n}_f16": (f"int{n}", 64, "f16") for n in (2, 3, 4, 5, 6, 8)},
}


def element_value(codes, elem: str) -> np.ndarray:
    if elem == "e2m1":
        return e2m1_value(codes)
    if elem == "e4m3":
        return e4m3_value(codes)
    if elem == "e5m2":
        return e5m2_value(codes)
    return int_value(codes, ELEMENTS[elem])


def scale_value(scales, kind: str) -> np.ndarray:
    """fp64 block scales as stored: E8M0 bytes, float32 or float16 arrays."""
    if kind == "e8m0":
        return e8m0_value(scales)
    if kind == "f32":
        return np.asarray(scales, dtype=np.float32).astype(np.float64)
    if kind == "f16":
        return np.asarray(scales, dtype=np.float16).astype(np.float64)
    raise ValueError(kind)


def implicit_factor(elem: str, kind: str) -> float:
    """2^-(n-2) for the mxint elements (see the module readings), else 1."""
    if elem.startswith("int") and kind == "e8m0":
        return 2.0 ** -(ELEMENTS[elem] - 2)
    return 1.0


def dequant_block(fmt: str, w_packed, scales, K: int) -> np.ndarray:
    """fp64 [N, K] weights of a Track-1 format: element(code) * factor *
    scale[block of k]."""
    elem, block, kind = FORMATS[fmt]
    codes = unpack_codes(np.asarray(w_packed, dtype=np.uint8), K, ELEMENTS[elem])
    val = element_value(codes, elem) * implicit_factor(elem, kind)
    s = scale_value(scales, kind)
    idx = np.arange(K) // block
    return val * s[:, idx]
