"""Bit layout and storage-dtype helpers of the oracle (fp64, NumPy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout of packed codes. "wh-iron kernel-op coverage audit", section
"Quantization precision coverage" (Track 1): sub-byte codes sit back to back,
least significant bit first (for 4-bit codes that is two codes per byte, the
low nibble first), and an 8-bit code takes one byte. The masks of `dequantize` / `qdot` in "mlx 1.0.0 -
quantized_nax.h" read every width (2/3/4/5/6/8) the same way: code j of a row
occupies bits [j*b, (j+1)*b) of the row's little-endian bit stream. The bytes
per row follow `get_pack_factor` / `get_bytes_per_pack` of the same listing:
K*b/8 bytes (3- and 5-bit codes come 8 per 3 or 5 bytes, 6-bit codes 4 per 3
bytes, the others 8/b per byte).

Here the stream is handled one bit at a time with NumPy's unpackbits /
packbits in little bit order; nothing here shares code with the library's
packer or with its GPU kernels.
"""

from __future__ import annotations

import numpy as np

_VALID_BITS = (2, 3, 4, 5, 6, 8)


def packed_row_bytes(K: int, bits: int) -> int:
    """Bytes of one packed row of K codes of `bits` bits (mlx quantized_nax.h,
    `get_pack_factor` / `get_bytes_per_pack`: K / pack_factor * bytes_per_pack)."""
    if bits not in _VALID_BITS:
        raise ValueError(f"bits must be one of {_VALID_BITS}, got {bits}")
    if (K * bits) % 8:
        raise ValueError("K*bits must be a whole number of bytes")
    return K * bits // 8


def unpack_codes(packed: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Codes [rows, K] (uint8) from packed rows [rows, K*bits/8] (uint8).

    Code j of a row is the integer whose bit i is bit (j*bits + i) of the row's
    little-endian bit stream (LSB-first packing, wh-iron audit Track 1)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    nb = packed_row_bytes(K, bits)
    if packed.shape[1] != nb:
        raise ValueError(f"packed rows must have {nb} bytes, got {packed.shape[1]}")
    stream = np.unpackbits(packed, axis=1, bitorder="little")  # [rows, K*bits]
    stream = stream.reshape(rows, K, bits).astype(np.uint32)
    place = (np.uint32(1) << np.arange(bits, dtype=np.uint32))
    return (stream * place).sum(axis=2).astype(np.uint8)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of `unpack_codes`: codes [rows, K] (each < 2**bits) -> packed
    rows [rows, K*bits/8], LSB-first."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    packed_row_bytes(K, bits)  # validates bits and K
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code does not fit in the given width")
    shifts = np.arange(bits, dtype=np.uint8)
    stream = (codes[:, :, None] >> shifts) & 1  # [rows, K, bits], bit i of code j
    return np.packbits(stream.reshape(rows, K * bits), axis=1, bitorder="little")


# --------------------------------------------------------------------------
# Storage dtypes. Activations, outputs and affine scales/biases are stored in
# one "T" of f32 / f16 / bf16 (mlx quantized_nax.h keeps x, scales, biases and
# y all in the kernel's T). bf16 is held as its raw uint16 bit pattern.
# --------------------------------------------------------------------------

def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored T data. bf16: the 16 stored bits are the top
    half of an IEEE binary32 pattern."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_f64_to_f32(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp64 -> fp32 (one rounding)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def round_f64_to_f16(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp64 -> fp16, directly from fp64 (NumPy converts
    double -> half without passing through single precision)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def round_f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp64 -> bfloat16, directly (no fp32 step, so no
    double rounding). Returns the uint16 bit patterns.

    bfloat16 keeps 8 significant bits and fp32's exponent range: the spacing
    of values in [2^e, 2^(e+1)) is 2^(e-7), and below 2^-126 it is the
    subnormal step 2^-133. Magnitudes that round to 2^128 or more overflow to
    infinity. NaN maps to the quiet NaN 0x7FC0 with its sign."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    fin = np.isfinite(v)
    vf = v[fin]
    _, ex = np.frexp(vf)               # |v| = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    step = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(vf / step) * step      # rint: halves go to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, vf), r)
    out[fin] = r
    out[~fin] = v[~fin]
    f32 = out.astype(np.float32)       # exact: every value is a bf16 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        sign = np.signbit(v[nan]).astype(np.uint16) << np.uint16(15)
        bits[nan] = sign | np.uint16(0x7FC0)
    return bits


def round_f64_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> stored T (RNE). bf16 comes back as uint16 bits."""
    if dtype == "f32":
        return round_f64_to_f32(v)
    if dtype == "f16":
        return round_f64_to_f16(v)
    if dtype == "bf16":
        return round_f64_to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def ulp_of(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of T values at each stored value (the gap to the next value
    away from zero; at zero and in the subnormal range it is T's smallest
    subnormal). Returned in fp64."""
    v = np.abs(storage_to_f64(stored, dtype))
    if dtype == "f32":
        mant, emin, sub = 23, -126, 2.0 ** -149
    elif dtype == "f16":
        mant, emin, sub = 10, -14, 2.0 ** -24
    elif dtype == "bf16":
        mant, emin, sub = 7, -126, 2.0 ** -133
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    out = np.full(v.shape, sub, dtype=np.float64)
    nz = (v > 0) & np.isfinite(v)
    _, ex = np.frexp(v[nz])
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    out[nz] = np.ldexp(1.0, (e - mant).astype(np.int32))
    return out
