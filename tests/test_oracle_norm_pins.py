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


def test_rms_factor_closed_forms():
    # (3, 4): r = 1 / sqrt(12.5); a constant row c with eps: 1 / sqrt(c^2 + eps)
    r = oracle.rms_factor(np.array([[3.0, 4.0], [0.5, 0.5]], np.float32), "f32", 0.0)
    assert r[0] == pytest.approx(1.0 / math.sqrt(12.5), rel=1e-15)
    assert r[1] == pytest.approx(2.0, rel=1e-15)
    r = oracle.rms_factor(np.full((1, 32), 0.5, np.float32), "f32", 0.25)
    assert r[0] == pytest.approx(1.0 / math.sqrt(0.5), rel=1e-15)


def test_rms_factor_times_gamma_product_is_the_norm():
    # r * (x * gamma) reproduces the plain RMSNorm row (to fp64 rounding)
    rng = np.random.default_rng(8)
    x = rng.normal(size=(2, 64)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, size=64).astype(np.float32)
    xn = oracle.rmsnorm(x, "f32", g, 1e-4)
    r = oracle.rms_factor(x, "f32", 1e-4)
    assert np.allclose(xn, r[:, None] * x.astype(np.float64) * g.astype(np.float64), rtol=1e-15)


def test_gamma_stored_identity_and_powers_of_two():
    rng = np.random.default_rng(9)
    x = oracle.round_f64_to(rng.normal(size=(2, 32)), "bf16")
    one = oracle.round_f64_to(np.ones(32), "bf16")
    assert np.array_equal(oracle.gamma_stored(x, "bf16", one), x)
    four = oracle.round_f64_to(np.full(32, 4.0), "bf16")
    assert np.array_equal(oracle.storage_to_f64(oracle.gamma_stored(x, "bf16", four), "bf16"),
                          4.0 * oracle.storage_to_f64(x, "bf16"))


def test_gamma_stored_matches_torch_rounding():
    # the product of two bf16 values is exact in fp32; torch's fp32 -> bf16
    # conversion (round to nearest even) must give the same stored values
    import torch
    rng = np.random.default_rng(10)
    xf = torch.from_numpy(rng.normal(size=(3, 64)).astype(np.float32)).to(torch.bfloat16)
    gf = torch.from_numpy(rng.uniform(0.3, 3.0, size=64).astype(np.float32)).to(torch.bfloat16)
    want = (xf.float() * gf.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = xf.view(torch.int16).numpy().view(np.uint16)
    g = gf.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.gamma_stored(x, "bf16", g), want)


def test_rmsnorm_qmv_closed_form_and_one_hot():
    # x = (3, 4), gamma = 1, eps = 0: xn = (0.6, 0.8) * sqrt(2); one-hot
    # weight rows pick each element, a row (1, -1) gives their difference
    W = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, -1.0], [2.0, 2.0]])
    y = oracle.rmsnorm_qmv(np.array([[3.0, 4.0]], np.float32), "f32", np.ones(2, np.float32),
                           0.0, W)
    s2 = math.sqrt(2.0)
    assert np.allclose(y[0], [0.6 * s2, 0.8 * s2, -0.2 * s2, 2.8 * s2], rtol=1e-15)
    A = oracle.rmsnorm_qmv_abs(np.array([[3.0, 4.0]], np.float32), "f32",
                               np.ones(2, np.float32), 0.0, W)
    assert np.allclose(A[0], [0.6 * s2, 0.8 * s2, 1.4 * s2, 2.8 * s2], rtol=1e-15)


def test_rmsnorm_qmv_brute_force_loops():
    # y[b, n] = sum_k W[n, k] x[b, k] r[b] gamma[k] by loops, bf16 storage,
    # W not square (a transposed operand fails on shape or value)
    rng = np.random.default_rng(11)
    B, K, N = 2, 6, 4
    x = oracle.round_f64_to(rng.normal(size=(B, K)), "bf16")
    g = oracle.round_f64_to(rng.uniform(0.5, 1.5, size=K), "bf16")
    W = rng.normal(size=(N, K))
    eps = 1e-2
    y = oracle.rmsnorm_qmv(x, "bf16", g, eps, W)
    A = oracle.rmsnorm_qmv_abs(x, "bf16", g, eps, W)
    X = oracle.storage_to_f64(x, "bf16")
    G = oracle.storage_to_f64(g, "bf16")
    assert y.shape == (B, N)
    for b in range(B):
        ms = sum(float(X[b, k]) ** 2 for k in range(K)) / K
        r = 1.0 / math.sqrt(ms + float(np.float32(eps)))
        for n in range(N):
            terms = [W[n, k] * X[b, k] * r * G[k] for k in range(K)]
            assert y[b, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-15)
            assert A[b, n] == pytest.approx(math.fsum(abs(t) for t in terms), rel=1e-13)


def test_rmsnorm_qmv_is_r_times_the_unrounded_gamma_product():
    # W . xn = r * (W . (x * gamma)) in exact arithmetic; the unrounded
    # product, not RN_T(x * gamma), is what the definition takes
    rng = np.random.default_rng(12)
    x = oracle.round_f64_to(rng.normal(size=(3, 64)), "f16")
    g = oracle.round_f64_to(rng.uniform(0.3, 3.0, size=64), "f16")
    W = rng.normal(size=(5, 64))
    y = oracle.rmsnorm_qmv(x, "f16", g, 1e-5, W)
    r = oracle.rms_factor(x, "f16", 1e-5)
    xg = oracle.storage_to_f64(x, "f16") * oracle.storage_to_f64(g, "f16")[None, :]
    assert np.allclose(y, r[:, None] * (xg @ W.T), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_staging_bound_admits_one_rounding_and_rejects_a_dropped_r(dtype):
    # the GPU tests' bound for the fused product (gpu_util.check_fused_norm):
    # a computation that rounds the staged activation once and the result
    # once, both to T, meets it; one that forgets r (a dropped term) does not
    import workloads
    from gpu_util import check_fused_norm
    rng = np.random.default_rng(13)
    B, K, N = 3, 1024, 200
    x = workloads.to_storage(3.0 * rng.normal(size=(B, K)), dtype)
    g = workloads.to_storage(rng.uniform(0.5, 1.5, size=K), dtype)
    W = rng.normal(size=(N, K)) * 0.05
    eps = 1e-6
    y_def = oracle.rmsnorm_qmv(x, dtype, g, eps, W)
    A_def = oracle.rmsnorm_qmv_abs(x, dtype, g, eps, W)
    xs = oracle.rmsnorm_stored(x, dtype, g, eps)           # the normalized row stored in T
    y_staged = oracle.round_f64_to(oracle.qmv(xs, dtype, W), dtype)
    check_fused_norm(y_staged, y_def, A_def, dtype, f"staged {dtype}")
    xg = oracle.gamma_stored(x, dtype, g)                   # r left out
    y_bad = oracle.round_f64_to(oracle.qmv(xg, dtype, W), dtype)
    with pytest.raises(AssertionError):
        check_fused_norm(y_bad, y_def, A_def, dtype, f"no r {dtype}")
