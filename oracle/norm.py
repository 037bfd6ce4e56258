"""RMSNorm in front of the QMV (the fused "RMSNorm + quantized GEMV").

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "wh-iron kernel-op coverage audit", the op-coverage rows "rms_norm"
and "rms_norm_qgemv (RMSNorm + quantized GEMV fused)", and the block-scaled
family's "fused RMSNorm + GEMV": a root-mean-square normalization of the
activation row, scaled per element by a weight vector, feeding the quantized
matrix-vector product in one dispatch.

Reading (the pages name the operation but print no formula): the usual
RMSNorm, xn[k] = x[k] * r * gamma[k] with r = 1 / sqrt(mean_k x^2 + eps) and
eps an argument, and the fused product is y = W . xn. `rmsnorm_qmv` is that
plain definition in fp64, with no intermediate rounding: the parity target.

A fused kernel has to hand the product a stored activation, so it rounds once
somewhere. `gamma_stored` and `rms_factor` describe one such choice (stage
RN_T(x * gamma), whose product of two T values is exact before the rounding,
and multiply the row's result by r); they serve as an extra, tighter check
of a kernel that makes that choice, never as the definition.
"""

from __future__ import annotations

import numpy as np

from .codes import round_f64_to, storage_to_f64


def rmsnorm(x, x_dtype: str, gamma, eps: float) -> np.ndarray:
    """fp64 xn[b, k] = x[b, k] * (1 / sqrt(mean_k x[b, k]^2 + eps)) * gamma[k]
    for stored x [B, K] and gamma [K] (eps taken as the fp32 the caller
    passes)."""
    x64 = storage_to_f64(x, x_dtype)
    if x64.ndim == 1:
        x64 = x64[None, :]
    g64 = storage_to_f64(gamma, x_dtype).reshape(-1)
    ms = np.mean(x64 * x64, axis=1)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    return x64 * r[:, None] * g64[None, :]


def rmsnorm_stored(x, x_dtype: str, gamma, eps: float) -> np.ndarray:
    """The normalized rows rounded to T (stored form), the QMV's input."""
    return round_f64_to(rmsnorm(x, x_dtype, gamma, eps), x_dtype)


def rms_factor(x, x_dtype: str, eps: float) -> np.ndarray:
    """fp64 r[b] = 1 / sqrt(mean_k x[b, k]^2 + eps) for stored x [B, K]."""
    x64 = storage_to_f64(x, x_dtype)
    if x64.ndim == 1:
        x64 = x64[None, :]
    return 1.0 / np.sqrt(np.mean(x64 * x64, axis=1) + float(np.float32(eps)))


def gamma_stored(x, x_dtype: str, gamma) -> np.ndarray:
    """RN_T(x[b, k] * gamma[k]) in stored form: what the fused product stages."""
    x64 = storage_to_f64(x, x_dtype)
    if x64.ndim == 1:
        x64 = x64[None, :]
    g64 = storage_to_f64(gamma, x_dtype).reshape(-1)
    return round_f64_to(x64 * g64[None, :], x_dtype)


def rmsnorm_qmv(x, x_dtype: str, gamma, eps: float, W64: np.ndarray) -> np.ndarray:
    """The fused product's plain definition in fp64: y[b, n] = sum_k
    W[n, k] * xn[b, k] with xn = rmsnorm(x) unrounded. W64 is the
    dequantized [N, K] matrix. Returns fp64 [B, N]."""
    return rmsnorm(x, x_dtype, gamma, eps) @ np.asarray(W64, dtype=np.float64).T


def rmsnorm_qmv_abs(x, x_dtype: str, gamma, eps: float, W64: np.ndarray) -> np.ndarray:
    """sum_k |W[n, k] * xn[b, k]| in fp64: the magnitude scale of each fused
    dot product (for error bounds)."""
    return np.abs(rmsnorm(x, x_dtype, gamma, eps)) @ np.abs(np.asarray(W64, np.float64)).T
