"""Pins for the projection Y = Q[(W - BA) D^(1/2)] (D^(-1/2) X) + B (A X)."""
import math

import numpy as np

import oracle
import workloads as wl


def _setup(seed, T=24, d=64, d_out=40, q=4, g=32, r=2, alpha=0.5):
    X = wl.gaussian(seed, (T, d), 2.0).astype(np.float16)
    W = wl.gaussian(seed + 1, (d_out, d), 0.05).astype(np.float16)
    D = oracle.colstats(X, alpha=alpha)
    B, A = oracle.svd_factors(W, r)
    c, s, z = oracle.quantize(oracle.residual(W, B, A), D, q, g)
    return X, W, D, B, A, c, s, z


def test_two_evaluations_agree():
    X, W, D, B, A, c, s, z = _setup(21)
    Y1 = oracle.linear(X, c, s, z, D, 32, B, A)
    Y2 = oracle.linear_dense(X, c, s, z, D, 32, B, A)
    np.testing.assert_allclose(Y1, Y2, rtol=1e-12, atol=1e-12 * np.abs(Y1).max())


def test_triple_loop_tiny():
    X, W, D, B, A, c, s, z = _setup(22, T=3, d=32, d_out=4, r=1)
    Y = oracle.linear(X, c, s, z, D, 32, B, A)
    for t in range(3):
        for i in range(4):
            acc = []
            for j in range(32):
                vh = (float(c[i, j]) - float(z[i, 0])) * float(s[i, 0])
                acc.append(vh * float(X[t, j]) / math.sqrt(float(D[j])))
                acc.append(float(B[i, 0]) * float(A[0, j]) * float(X[t, j]))
            assert abs(Y[t, i] - math.fsum(acc)) <= 1e-12 * max(1.0, abs(Y[t, i]))


def test_exactly_representable_weight_gives_exact_product():
    """If W D^(1/2) already lies on every group's grid, the quantiser is
    lossless and Y = X W^T exactly (checks the D^(1/2) scaling in the quantiser
    against the D^(-1/2) pre-scaling of the input)."""
    rng = np.random.default_rng(5)
    d, d_out, g, q = 64, 8, 32, 4
    D = np.full(d, 4.0, np.float32)                       # sqrt(D) = 2
    codes = rng.integers(0, 16, size=(d_out, d))
    codes[:, ::g] = 0                                     # every group spans 0 .. 15
    codes[:, 1::g] = 15
    zc = 5
    v = (codes - zc) * 0.25                               # grid with s = 0.25, z = 5
    W = (v / 2.0).astype(np.float16)                      # W D^(1/2) = v exactly
    c, s, z = oracle.quantize(W, D, q, g)
    assert np.all(s == 0.25) and np.all(z == zc)
    X = wl.gaussian(6, (5, d), 1.0)
    Y = oracle.linear(X, c, s, z, D, g)
    np.testing.assert_allclose(Y, X @ W.astype(np.float64).T, rtol=1e-13, atol=1e-13)


def test_alpha0_rank0_is_rtn_layer():
    X, W, D, B, A, c, s, z = _setup(23, r=0, alpha=0.0)
    assert np.all(D == 1)
    Y = oracle.linear(X, c, s, z, D, 32)
    Wh = oracle.dequant(c, s, z, 32)
    np.testing.assert_allclose(Y, X.astype(np.float64) @ Wh.T, rtol=1e-13)


def test_quantised_layer_close_to_full_precision():
    X, W, D, B, A, c, s, z = _setup(24, q=4, r=0)
    Y = oracle.linear(X, c, s, z, D, 32)
    Yf = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(Y - Yf) / np.linalg.norm(Yf) < 0.1
    # full-rank factors leave a zero residual: Y is the full-precision layer
    B, A = oracle.svd_factors(W, 40)
    R = oracle.residual(W, B, A)
    c, s, z = oracle.quantize(R, D, 4, 32)
    Y2 = oracle.linear(X, c, s, z, D, 32, B, A)
    assert np.linalg.norm(Y2 - Yf) / np.linalg.norm(Yf) < 1e-3
