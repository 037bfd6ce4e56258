"""Fused routed-MoE decode block: gate/up projections with the SwiGLU
activation, then the down projection summed over each token's routed experts
with the router weights folded in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "@lgrammel/ds4-provider - moe.metal", the routed-MoE activation kernels and
  the fused gate/up + activation decode kernel: for each routed slot,
  mid = silu(g) * u with silu(g) = g / (1 + exp(-g)), where g and u are the
  slot's gate and up projections, each first clamped when a positive clamp
  value c is configured (g = min(g, c), u = clamp(u, -c, c)); and the down
  kernel that loops over a token's expert slots, accumulating their
  projections into one output row.
* "wh-iron kernel-op coverage audit", op-coverage row "moe routed-expert
  decode fuse": the block runs as two dispatches, per-(slot, tile) gate/up QMV
  with the activation in its epilogue, then a down QMV over the top_k slots of
  each token that folds in the router weights.

Readings (where the pages leave a step open): mid is stored in the activation
dtype T (rounded to nearest even); the router weights are fp32 inputs, applied
in the down step as y[t] = sum_j r[t, j] * (W_down[e[t, j]] @ mid[t, j]); a slot
whose expert id is out of range contributes nothing (its mid row is zero).
Everything here is fp64 from the stored inputs.
"""

from __future__ import annotations

import numpy as np

from .codes import storage_to_f64


def silu(g):
    """silu(g) = g / (1 + exp(-g)) in fp64 (for g < -700 exp overflows to inf
    and the quotient is -0.0 or 0, the correct limit)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g, u, clamp: float = 0.0):
    """The activation of one slot: optional clamp, then silu(g) * u (fp64)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    if clamp > 1e-6:
        g = np.minimum(g, clamp)
        u = np.clip(u, -clamp, clamp)
    return silu(g) * u


def gate_up_projections(x, x_dtype: str, expert_ids, n_experts: int, Wg_of, Wu_of):
    """fp64 gate and up projections of every slot s = t * top_k + j:
    g[s] = W_gate[e] @ x[t], u[s] = W_up[e] @ x[t] with e = expert_ids[t, j];
    rows of slots with an out-of-range expert are zero. Wg_of(e) / Wu_of(e)
    return the fp64 dequantized [ffn, hidden] matrices."""
    x64 = storage_to_f64(x, x_dtype)
    ids = np.asarray(expert_ids, dtype=np.int64)
    T, k = ids.shape
    ffn = Wg_of(0).shape[0]
    g = np.zeros((T * k, ffn))
    u = np.zeros((T * k, ffn))
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < n_experts:
                continue
            if e not in cache:
                cache[e] = (Wg_of(e), Wu_of(e))
            Wg, Wu = cache[e]
            g[t * k + j] = Wg @ x64[t]
            u[t * k + j] = Wu @ x64[t]
    return g, u


def moe_gate_up_swiglu(x, x_dtype: str, expert_ids, n_experts: int, Wg_of, Wu_of,
                       clamp: float = 0.0):
    """mid[s] = swiglu(g[s], u[s]) in fp64 ([T * top_k, ffn]); out-of-range
    slots give zero rows."""
    g, u = gate_up_projections(x, x_dtype, expert_ids, n_experts, Wg_of, Wu_of)
    ids = np.asarray(expert_ids, dtype=np.int64).reshape(-1)
    mid = swiglu(g, u, clamp)
    mid[(ids < 0) | (ids >= n_experts)] = 0.0
    return mid


def moe_down_reduce(mid, mid_dtype: str, expert_ids, route_weights, n_experts: int, Wd_of):
    """y[t] = sum_j r[t, j] * (W_down[e[t, j]] @ mid[t * top_k + j]) in fp64,
    from the stored mid rows; slots with an out-of-range expert add nothing.
    Returns (y [T, hidden], the fp64 sum of |terms| per output for error
    bounds)."""
    m64 = storage_to_f64(mid, mid_dtype)
    ids = np.asarray(expert_ids, dtype=np.int64)
    r = np.asarray(route_weights, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    hidden = Wd_of(0).shape[0]
    y = np.zeros((T, hidden))
    a = np.zeros((T, hidden))
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < n_experts:
                continue
            if e not in cache:
                cache[e] = Wd_of(e)
            Wd = cache[e]
            v = m64[t * k + j]
            y[t] += r[t, j] * (Wd @ v)
            a[t] += abs(r[t, j]) * (np.abs(Wd) @ np.abs(v))
    return y, a
