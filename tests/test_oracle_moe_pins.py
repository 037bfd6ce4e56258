"""Pins of the fused routed-MoE oracle: the activation against SciPy's logistic
function, the clamp, and the two projections reduced to the gather / QMV
oracle (itself pinned elsewhere) or to exact small-integer arithmetic."""

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads


def test_silu_matches_logistic_times_input():
    g = np.concatenate([np.linspace(-60, 60, 2001), [0.0, 1e-300, -1e-300]])
    want = g * expit(g)
    got = oracle.silu(g)
    assert np.allclose(got, want, rtol=4e-16, atol=0)


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(50.0) == 50.0                   # 1 + e^-50 rounds to 1
    assert oracle.silu(-800.0) == 0.0                  # exp overflows: the limit 0
    assert np.isclose(oracle.silu(-30.0), -30.0 * np.exp(-30.0) / (1 + np.exp(-30.0)),
                      rtol=1e-15)


def test_swiglu_clamp():
    c = 1.5
    g = np.array([5.0, -5.0, 0.5])
    u = np.array([-3.0, 2.0, 0.25])
    got = oracle.swiglu(g, u, clamp=c)
    want = oracle.silu(np.array([1.5, -5.0, 0.5])) * np.array([-1.5, 1.5, 0.25])
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.swiglu(g, u), oracle.silu(g) * u)   # no clamp


def _moe_small(top_k=3, T=4, E=6, ffn=64, hidden=96, seed=0):
    rng = np.random.default_rng(seed)
    Wg = rng.integers(-3, 4, size=(E, ffn, hidden)).astype(np.float64)
    Wu = rng.integers(-3, 4, size=(E, ffn, hidden)).astype(np.float64)
    Wd = rng.integers(-3, 4, size=(E, hidden, ffn)).astype(np.float64)
    x = rng.integers(-4, 5, size=(T, hidden)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:top_k] for _ in range(T)]).astype(np.uint32)
    return Wg, Wu, Wd, x, ids


def test_gate_up_projections_equal_gather_oracle():
    Wg, Wu, Wd, x, ids = _moe_small()
    T, k = ids.shape
    g, u = oracle.gate_up_projections(x, "f32", ids, 6, lambda e: Wg[e], lambda e: Wu[e])
    lhs = (np.arange(T * k) // k).astype(np.uint32)
    rhs = ids.reshape(-1)
    gg = oracle.gather_qmv(x, "f32", lhs, rhs, 6, Wg.shape[1], lambda e: Wg[e])
    uu = oracle.gather_qmv(x, "f32", lhs, rhs, 6, Wu.shape[1], lambda e: Wu[e])
    assert np.array_equal(g, gg) and np.array_equal(u, uu)


def test_gate_up_out_of_range_slot_is_zero():
    Wg, Wu, Wd, x, ids = _moe_small()
    ids = ids.copy()
    ids[1, 2] = 99
    mid = oracle.moe_gate_up_swiglu(x, "f32", ids, 6, lambda e: Wg[e], lambda e: Wu[e])
    assert not mid[1 * 3 + 2].any()
    assert mid[0].any()


def test_down_reduce_exact_small_integers():
    # integer weights, integer mid values, router weights powers of two:
    # every product and sum is exact in fp64, so y is the integer result
    Wg, Wu, Wd, x, ids = _moe_small()
    T, k = ids.shape
    rng = np.random.default_rng(1)
    mid = rng.integers(-5, 6, size=(T * k, Wd.shape[2])).astype(np.float32)
    r = np.ldexp(1.0, rng.integers(-3, 2, size=(T, k))).astype(np.float32)
    y, a = oracle.moe_down_reduce(mid, "f32", ids, r, 6, lambda e: Wd[e])
    exact = np.zeros((T, Wd.shape[1]))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            exact[t] += float(r[t, j]) * (Wd[e].astype(np.int64) @ mid[t * k + j].astype(np.int64))
    assert np.array_equal(y, exact)
    assert (a >= np.abs(y)).all()


def test_down_reduce_top1_unit_weight_is_qmv():
    Wg, Wu, Wd, x, ids = _moe_small(top_k=1)
    T = ids.shape[0]
    rng = np.random.default_rng(2)
    mid = workloads.to_storage(rng.normal(size=(T, Wd.shape[2])), "bf16")
    y, _ = oracle.moe_down_reduce(mid, "bf16", ids, np.ones((T, 1), np.float32), 6,
                                  lambda e: Wd[e])
    for t in range(T):
        assert np.array_equal(y[t], oracle.qmv(mid[t:t + 1], "bf16", Wd[int(ids[t, 0])])[0])


def test_down_reduce_linear_in_router_weights():
    Wg, Wu, Wd, x, ids = _moe_small()
    rng = np.random.default_rng(3)
    mid = rng.normal(size=(12, Wd.shape[2])).astype(np.float32)
    r = rng.random((4, 3)).astype(np.float32)
    y1, _ = oracle.moe_down_reduce(mid, "f32", ids, r, 6, lambda e: Wd[e])
    y2, _ = oracle.moe_down_reduce(mid, "f32", ids, 2 * r, 6, lambda e: Wd[e])
    assert np.array_equal(y2, 2 * y1)
