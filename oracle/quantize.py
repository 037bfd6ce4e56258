"""Quantize-from-float: the encoders that turn a float weight matrix into the
packed formats this library multiplies.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name these encoders without fixing every step, so each function
states the reading it implements (the same readings are listed with the rest
of the design):

* "wh-iron kernel-op coverage audit", section "Quantization precision
  coverage", Track 2 and its closing bullets: the affine integer track is
  encoded by a cheap per-group min/max giving a scale and a bias
  (w = scale*q + bias). Reading: scale = (max - min) / (2^b - 1), bias = min,
  both stored in the weight dtype T; codes are taken against the *stored*
  scale and bias, rounded half to even and clamped to [0, 2^b - 1].
* Same audit, op-coverage rows fp_quantized and kv_cache: the float formats
  take a per-block maximum as the scale and round each element to the nearest
  representable value, saturating (no NaN or infinity produced). Reading for
  the MX formats (OCP MX construction): the E8M0 block exponent is
  floor(log2(amax)) minus the element's largest exponent (2 for E2M1, whose
  largest value is 1.5*2^2; 8 for E4M3, 1.75*2^8), clamped to the byte range;
  an all-zero block takes byte 0.
* Same audit, Track-1 format table (nvfp4: E2M1 elements, E4M3 scale per 16,
  tensor-wide fp32 global). Reading for the two levels: global =
  amax(tensor) / (448 * 6), so the largest block scale lands on E4M3's
  largest value; block scale = E4M3 nearest to amax(block) / 6 / global;
  elements = E2M1 nearest to w / (block scale * global).

Every arithmetic step that decides a code is a single fp32 operation here
(NumPy float32 arithmetic rounds each operation to nearest even), written in
the order stated, so an implementation that performs the same fp32 steps
reaches the same codes. Element rounding is defined by nearest-value search
over the format's values, not by bit manipulation.
"""

from __future__ import annotations

import numpy as np

from .codes import storage_to_f64
from .formats import e2m1_value, e4m3_value, e4m3_encode_nearest, nearest_code

_F32 = np.float32

_E2M1_POS_VALUES = e2m1_value(np.arange(8))          # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode_nearest(v) -> np.ndarray:
    """E2M1 code (uint8, 0..15) nearest to v: the nearest of the 8 magnitudes
    wins; an exact tie goes to the even code (mantissa bit 0); magnitudes above
    6 saturate to 6 (code 7); the sign (including that of -0.0) goes to bit 3."""
    v = np.asarray(v, dtype=np.float64)
    code = nearest_code(np.minimum(np.abs(v), 6.0), _E2M1_POS_VALUES).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(8), code).astype(np.uint8)


def _to_f32(w_stored, dtype: str) -> np.ndarray:
    """Stored T values widened to fp32 (exact for f32 / f16 / bf16)."""
    return storage_to_f64(w_stored, dtype).astype(np.float32)


def _store(v32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> stored T with one round-to-nearest-even (bf16 as uint16 bits)."""
    v32 = np.asarray(v32, dtype=np.float32)
    if dtype == "f32":
        return v32.copy()
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return v32.astype(np.float16)
    if dtype == "bf16":
        b = v32.view(np.uint32).astype(np.uint64)
        r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        out = r.astype(np.uint16)
        nan = np.isnan(v32)
        out[nan] = (out[nan] & 0x8000) | 0x7FC0
        return out
    raise ValueError(dtype)


def floor_log2(a) -> np.ndarray:
    """floor(log2(a)) for positive finite a (fp32 values, subnormals included),
    via the exact fp64 frexp: a = m * 2^e with m in [0.5, 1)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def quantize_affine(w_stored, dtype: str, bits: int, group: int):
    """Affine (Track 2) encoder of a [N, K] matrix in T.

    Per group of `group` consecutive elements of a row, in fp32:
      lo, hi = min, max of the group (each + 0, so a zero extreme is +0)
      s32 = (hi - lo) / (2^bits - 1)            (two fp32 operations)
      stored scale = RN_T(s32), stored bias = RN_T(lo)
      s, b = the stored values widened back to fp32
      q = 0 if s == 0, else clamp(rint_even((w - b) / s), 0, 2^bits - 1)
    Returns (codes uint8 [N, K], scales [N, K/group] as stored T, biases)."""
    v = _to_f32(w_stored, dtype)
    N, K = v.shape
    n = _F32(2 ** bits - 1)
    g = v.reshape(N, K // group, group)
    lo = g.min(axis=2) + _F32(0)      # -0 + 0 = +0: zero extremes count as +0
    hi = g.max(axis=2) + _F32(0)
    s32 = (hi - lo) / n
    s_st = _store(s32, dtype)
    b_st = _store(lo, dtype)
    s = _to_f32(s_st, dtype)[:, :, None]
    b = _to_f32(b_st, dtype)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - b) / np.where(s == 0, _F32(1), s)
    q = np.clip(np.rint(t), 0, float(n))
    q = np.where(s == 0, 0, q).astype(np.uint8)
    return q.reshape(N, K), s_st, b_st


_EMAX = {"e2m1": 2, "e4m3": 8}


def _encode(elem: str, t) -> np.ndarray:
    return e2m1_encode_nearest(t) if elem == "e2m1" else e4m3_encode_nearest(t)


def quantize_mx(w_stored, dtype: str, elem: str):
    """MX encoder (block 32, E8M0 scale) of a [N, K] matrix in T; elem is
    'e2m1' (MXFP4) or 'e4m3' (MXFP8).

    Per block of 32 in fp32: a = max |w|; byte = 0 if a == 0, else
    clamp(floor(log2 a) - emax + 127, 0, 254); X = 2^(byte - 127);
    code_j = nearest element to w_j / X (ties to even, saturating; sign from w).
    Returns (codes uint8 [N, K], E8M0 bytes [N, K/32])."""
    v = _to_f32(w_stored, dtype)
    N, K = v.shape
    blk = v.reshape(N, K // 32, 32)
    a = np.abs(blk).max(axis=2)
    e = np.where(a > 0, floor_log2(np.where(a > 0, a, 1)) - _EMAX[elem] + 127, 0)
    byte = np.clip(e, 0, 254).astype(np.uint8)
    X = np.ldexp(np.float32(1.0), byte.astype(np.int32) - 127).astype(np.float32)
    t = blk / X[:, :, None]
    codes = _encode(elem, t).reshape(N, K)
    return codes, byte


NV_GLOBAL_DIV = np.float32(448.0 * 6.0)


def quantize_nvfp4(w_stored, dtype: str):
    """NVFP4 two-level encoder of a [N, K] matrix in T.

    In fp32: A = max |w| over the matrix; global = A / 2688 (= 448 * 6).
    Per block of 16: sb = (max |w| / 6) / global (two operations; 0 when
    global is 0); scale byte = E4M3 nearest to sb (saturating at 448);
    d = decoded scale * global; code_j = E2M1 nearest to w_j / d (code 0 when
    d is 0). Returns (codes uint8 [N, K], E4M3 bytes [N, K/16], global fp32)."""
    v = _to_f32(w_stored, dtype)
    N, K = v.shape
    A = np.abs(v).max() if v.size else np.float32(0)
    gs = np.float32(A) / NV_GLOBAL_DIV
    blk = v.reshape(N, K // 16, 16)
    ab = np.abs(blk).max(axis=2)
    if gs > 0:
        sb = (ab / np.float32(6.0)) / gs
    else:
        sb = np.zeros_like(ab)
    byte = e4m3_encode_nearest(sb).reshape(ab.shape)
    d = (e4m3_value(byte).astype(np.float32) * gs).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = blk / np.where(d == 0, np.float32(1), d)[:, :, None]
    codes = e2m1_encode_nearest(t).reshape(N, K // 16, 16)
    codes = np.where((d == 0)[:, :, None], 0, codes).astype(np.uint8)
    return codes.reshape(N, K), byte, np.float32(gs)
