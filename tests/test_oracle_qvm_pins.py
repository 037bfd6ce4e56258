"""Pins of the qvm oracle: one-hot x picks out one dequantized row (layout and
indexing), an exact small-integer case worked element by element in the
`qouter` form x * (s*q + b), and the transpose relation to the QMV oracle."""

import math

import numpy as np

import oracle
import workloads


def test_qvm_one_hot_selects_dequantized_row():
    c = workloads.affine_case(9, "qvm-pin", bits=4, group=64, K=256, N=40, B=1, dtype="f32")
    W = oracle.dequant("affine", c.K, c.w, c.scales, c.biases, 4, 64, "f32")
    for n in (0, 7, 39):
        x = np.zeros((1, c.N), np.float32)
        x[0, n] = 1.0
        assert np.array_equal(oracle.qvm(x, "f32", W)[0], W[n])


def test_qvm_exact_qouter_form():
    # integer codes, power-of-two scales, integer biases: every term exact
    rng = np.random.default_rng(0)
    N, K, g = 6, 64, 32
    q = rng.integers(0, 16, size=(N, K))
    s = np.ldexp(1.0, rng.integers(-3, 2, size=(N, K // g)))
    b = rng.integers(-4, 5, size=(N, K // g)).astype(np.float64)
    x = rng.integers(-3, 4, size=(2, N)).astype(np.float32)
    w = oracle.pack_codes(q.astype(np.uint8), 4)
    W = oracle.dequant("affine", K, w, s.astype(np.float32), b.astype(np.float32), 4, g, "f32")
    y = oracle.qvm(x, "f32", W)
    for bb in range(2):
        for k in range(K):
            acc = 0.0
            for n in range(N):
                acc += float(x[bb, n]) * (s[n, k // g] * q[n, k] + b[n, k // g])
            assert y[bb, k] == acc


def test_qvm_is_qmv_of_the_transpose():
    rng = np.random.default_rng(1)
    W = rng.normal(size=(50, 96))
    x = workloads.to_storage(rng.normal(size=(3, 50)), "bf16")
    assert np.allclose(oracle.qvm(x, "bf16", W), oracle.qmv(x, "bf16", W.T), rtol=1e-13, atol=0)


def test_qvm_abs_brute_force():
    # sum_n |x[b, n] * W[n, k]| by loops; negative x and W, and a non-square
    # W, so a dropped absolute value or a transposed operand fails
    rng = np.random.default_rng(2)
    N, K = 7, 12
    W = rng.normal(size=(N, K))
    x = workloads.to_storage(rng.normal(size=(3, N)), "f16")
    X = oracle.storage_to_f64(x, "f16")
    A = oracle.qvm_abs(x, "f16", W)
    assert A.shape == (3, K)
    for b in range(3):
        for k in range(K):
            want = sum(abs(X[b, n] * W[n, k]) for n in range(N))
            assert math.isclose(A[b, k], want, rel_tol=1e-14), (b, k)
    # it bounds the product, with equality where every term has one sign
    assert np.all(np.abs(oracle.qvm(x, "f16", W)) <= A * (1 + 1e-14))
    xp = workloads.to_storage(np.abs(rng.normal(size=(2, N))), "bf16")
    Wp = np.abs(W)
    assert np.allclose(oracle.qvm(xp, "bf16", Wp), oracle.qvm_abs(xp, "bf16", Wp),
                       rtol=1e-15, atol=0)
