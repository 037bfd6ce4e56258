"""Dequantization and the quantized matrix-vector product, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method reaches, up to fp32 rounding order, the plain result
y = x . dequant(W)^T, so this module is that definition written out: decode
every element of W to fp64 from its format's definition, then one fp64 matrix
product. No blocking, no Sigma-x factoring, no fusion.

Layouts (row-major, contiguous):
  x       [B, K]   stored T (f32 / f16 / bf16 as uint16 bits)
  affine  w [N, K*bits/8] uint8, scales / biases [N, K/group] stored T
  mxfp4   w [N, K/2] uint8 (E2M1, even k in the low nibble), scales [N, K/32] E8M0
  nvfp4   w [N, K/2] uint8 (E2M1), scales [N, K/16] E4M3, global fp32 scalar
  mxfp8   w [N, K]   uint8 (E4M3), scales [N, K/32] E8M0
"""

from __future__ import annotations

import numpy as np

from .codes import unpack_codes, storage_to_f64
from .formats import e2m1_value, e4m3_value, e8m0_value


def _block_index(K: int, block: int) -> np.ndarray:
    return np.arange(K) // block


def dequant_affine(w, scales, biases, K: int, bits: int, group: int, dtype: str) -> np.ndarray:
    """Affine ("Track 2" of the wh-iron audit) weights: w = scale * q + bias per
    group of `group` consecutive k, q the unsigned `bits`-bit code (mlx
    quantized_nax.h `dequantize`). Returns fp64 [N, K]."""
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    q = unpack_codes(w, K, bits).astype(np.float64)
    g = _block_index(K, group)
    s = storage_to_f64(scales, dtype)[:, g]
    b = storage_to_f64(biases, dtype)[:, g]
    return s * q + b


def dequant_mxfp4(w, scales, K: int) -> np.ndarray:
    """MXFP4 (wh-iron audit Track-1 table): E2M1 element times the E8M0 scale
    of its block of 32. Returns fp64 [N, K]."""
    codes = unpack_codes(w, K, 4)
    return e2m1_value(codes) * e8m0_value(np.asarray(scales))[:, _block_index(K, 32)]


def dequant_nvfp4(w, scales, K: int, global_scale: float | None) -> np.ndarray:
    """NVFP4 (wh-iron audit Track-1 table): E2M1 element times the E4M3 scale of
    its block of 16 times the tensor-wide fp32 global scale (1.0 when absent;
    mlx pull request 4516 covers NVFP4 calls with and without one)."""
    codes = unpack_codes(w, K, 4)
    g = 1.0 if global_scale is None else float(np.float32(global_scale))
    return e2m1_value(codes) * e4m3_value(np.asarray(scales))[:, _block_index(K, 16)] * g


def dequant_mxfp8(w, scales, K: int) -> np.ndarray:
    """MXFP8 with E4M3 elements (wh-iron audit Track-1 table, mxfp8_e4m3):
    E4M3 element times the E8M0 scale of its block of 32."""
    codes = np.asarray(w, dtype=np.uint8)
    if codes.shape[1] != K:
        raise ValueError("mxfp8 rows hold one byte per element")
    return e4m3_value(codes) * e8m0_value(np.asarray(scales))[:, _block_index(K, 32)]


def dequant(fmt: str, K: int, w, scales, biases=None, bits: int = 4, group: int = 64,
            dtype: str = "f32", global_scale=None) -> np.ndarray:
    """Dispatch on the format name: 'affine', 'mxfp4', 'nvfp4', 'mxfp8'."""
    if fmt == "affine":
        return dequant_affine(w, scales, biases, K, bits, group, dtype)
    if fmt == "mxfp4":
        return dequant_mxfp4(w, scales, K)
    if fmt == "nvfp4":
        return dequant_nvfp4(w, scales, K, global_scale)
    if fmt == "mxfp8":
        return dequant_mxfp8(w, scales, K)
    from .blockfmt import FORMATS, dequant_block
    if fmt in FORMATS:
        return dequant_block(fmt, w, scales, K)
    raise ValueError(f"unknown format {fmt!r}")


def qmv(x, x_dtype: str, W64: np.ndarray) -> np.ndarray:
    """y[b, n] = sum_k x[b, k] * W[n, k] in fp64 (x given as stored T data,
    W already dequantized to fp64). Returns fp64 [B, N]."""
    x64 = storage_to_f64(x, x_dtype)
    if x64.ndim == 1:
        x64 = x64[None, :]
    return x64 @ W64.T


def qmv_rows(fmt: str, x, x_dtype: str, K: int, rows, w, scales, biases=None,
             bits: int = 4, group: int = 64, global_scale=None) -> np.ndarray:
    """The same product restricted to the output rows `rows` (for spot checks
    of full-size problems): only those weight rows are decoded. Returns fp64
    [B, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    w_sel = np.asarray(w)[rows]
    s_sel = np.asarray(scales)[rows]
    b_sel = None if biases is None else np.asarray(biases)[rows]
    W64 = dequant(fmt, K, w_sel, s_sel, b_sel, bits=bits, group=group,
                  dtype=x_dtype, global_scale=global_scale)
    return qmv(x, x_dtype, W64)


def gather_qmv(x, x_dtype: str, lhs_indices, rhs_indices, n_experts: int, N: int,
               W64_of_expert) -> np.ndarray:
    """Routed-expert gather: y[s] = W[rhs[s]] . x[lhs[s]] for every slot s.

    Semantics of `adjust_matrix_offsets` in mlx quantized_nax.h (x row chosen
    by lhs_indices, weight matrix by rhs_indices) and of `kernel_mul_mv_id` in
    the ds4-provider moe.metal listing (the expert id of each slot picks the
    weights). An index out of range (x row >= number of x rows, or expert >=
    n_experts) gives a row of zeros, the convention of the ferrum-kernels
    primitives.rs tests for out-of-range ids.

    `W64_of_expert` is a callable e -> fp64 [N, K], so only the experts in use
    get decoded. Returns fp64 [n_slots, N]."""
    x64 = storage_to_f64(x, x_dtype)
    if x64.ndim == 1:
        x64 = x64[None, :]
    lhs = np.asarray(lhs_indices, dtype=np.int64)
    rhs = np.asarray(rhs_indices, dtype=np.int64)
    out = np.zeros((lhs.shape[0], N), dtype=np.float64)
    cache = {}
    for s in range(lhs.shape[0]):
        e, r = int(rhs[s]), int(lhs[s])
        if not (0 <= e < n_experts and 0 <= r < x64.shape[0]):
            continue
        if e not in cache:
            cache[e] = W64_of_expert(e)
        out[s] = cache[e] @ x64[r]
    return out


def abs_dot(x, x_dtype: str, W64: np.ndarray) -> np.ndarray:
    """A[b, n] = sum_k |x[b, k] * W[n, k]| in fp64: the magnitude scale of each
    dot product, used to recognise outputs that are small only through
    cancellation."""
    x64 = np.abs(storage_to_f64(x, x_dtype))
    if x64.ndim == 1:
        x64 = x64[None, :]
    return x64 @ np.abs(W64).T


def qvm(x, x_dtype: str, W64: np.ndarray) -> np.ndarray:
    """The transposed product y[b, k] = sum_n x[b, n] * W[n, k] in fp64, with W
    the [N, K] dequantized matrix in the same packed layout the QMV reads
    ("mlx 1.0.0 - quantized_nax.h", `qouter`: each row n adds x[n] times its
    dequantized row, scale*q + bias per element). x is [B, N]."""
    return storage_to_f64(x, x_dtype) @ np.asarray(W64, dtype=np.float64)


def qvm_abs(x, x_dtype: str, W64: np.ndarray) -> np.ndarray:
    """sum_n |x[b, n] * W[n, k]| (for error bounds)."""
    return np.abs(storage_to_f64(x, x_dtype)) @ np.abs(np.asarray(W64, dtype=np.float64))
