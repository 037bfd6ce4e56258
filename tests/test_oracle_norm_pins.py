"""Pins of the RMSNorm oracle against closed forms, invariants and explicit
loops (none of them restates the vectorized formula)."""

import math

import numpy as np
import pytest

import oracle


def test_three_four_closed_form():
    # mean of squares of (3, 4) is 12.5; with eps = 0 and gamma = 1 the row
    # becomes (3, 4) / sqrt(12.5) = (0.6, 0.8) * sqrt(2)
    xn = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), "f32", np.ones(2, np.float32), 0.0)
    assert np.allclose(xn[0], [0.6 * math.sqrt(2.0), 0.8 * math.sqrt(2.0)], rtol=1e-15)


def test_constant_row_and_eps():
    # a constant row c gives c / sqrt(c^2 + eps) everywhere
    c, eps = 0.5, 0.25
    x = np.full((1, 64), c, np.float32)
    xn = oracle.rmsnorm(x, "f32", np.ones(64, np.float32), eps)
    assert np.allclose(xn, c / math.sqrt(c * c + eps), rtol=1e-15)


def test_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 96)).astype(np.float32)
    g = np.ones(96, np.float32)
    xn = oracle.rmsnorm(x, "f32", g, 0.0)
    assert np.allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-13)
    # with eps = 0, scaling a row by a power of two changes nothing
    xn2 = oracle.rmsnorm(x * np.float32(8.0), "f32", g, 0.0)
    assert np.allclose(xn, xn2, rtol=1e-14)


def test_gamma_multiplies_elementwise_brute_force():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(2, 5)).astype(np.float32)
    g = rng.uniform(0.5, 2.0, size=5).astype(np.float32)
    eps = 1e-3
    xn = oracle.rmsnorm(x, "f32", g, eps)
    for b in range(2):
        s = 0.0
        for k in range(5):
            s += float(x[b, k]) ** 2
        r = 1.0 / math.sqrt(s / 5 + float(np.float32(eps)))
        for k in range(5):
            assert xn[b, k] == pytest.approx(float(x[b, k]) * r * float(g[k]), rel=1e-14)


def test_stored_rounding_is_round_to_nearest():
    # bf16 storage of the normalized row is the nearest bf16 value
    rng = np.random.default_rng(7)
    x = oracle.round_f64_to(rng.normal(size=(1, 64)), "bf16")
    g = oracle.round_f64_to(rng.uniform(0.5, 1.5, size=64), "bf16")
    xn = oracle.rmsnorm(x, "bf16", g, 1e-6)
    st = oracle.storage_to_f64(oracle.rmsnorm_stored(x, "bf16", g, 1e-6), "bf16")
    ulp = oracle.ulp_of(oracle.rmsnorm_stored(x, "bf16", g, 1e-6), "bf16")
    assert np.all(np.abs(st - xn) <= ulp / 2)
