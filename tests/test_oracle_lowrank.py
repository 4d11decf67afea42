"""Pins for the static low-rank factors and the residual."""
import numpy as np
import scipy.linalg

import oracle
import workloads as wl


def test_eckart_young():
    # ||W - B A||_F^2 equals the sum of the trailing squared singular values,
    # taken here from the eigenvalues of W^T W (a different LAPACK routine)
    W = wl.gaussian(11, (96, 64), 0.02).astype(np.float16)
    W64 = W.astype(np.float64)
    sig2 = np.sort(scipy.linalg.eigvalsh(W64.T @ W64))[::-1]
    for r in (1, 4, 16):
        B, A = oracle.svd_factors(W, r)
        assert B.shape == (96, r) and A.shape == (r, 64)
        resid = np.linalg.norm(W64 - B.astype(np.float64) @ A.astype(np.float64)) ** 2
        np.testing.assert_allclose(resid, sig2[r:].sum(), rtol=1e-5)


def test_full_rank_reproduces_W():
    W = wl.gaussian(12, (40, 32), 0.05).astype(np.float16)
    B, A = oracle.svd_factors(W, 32)
    W64 = W.astype(np.float64)
    rel = np.linalg.norm(W64 - B.astype(np.float64) @ A.astype(np.float64)) / np.linalg.norm(W64)
    assert rel <= 1e-5


def test_balanced_split():
    W = wl.gaussian(13, (50, 30), 1.0)
    B, A = oracle.svd_factors(W, 5)
    # columns of B and rows of A carry equal norms (sqrt of each singular value)
    np.testing.assert_allclose(np.linalg.norm(B, axis=0), np.linalg.norm(A, axis=1), rtol=1e-5)


def test_rank_zero_is_identity():
    W = wl.gaussian(14, (8, 32), 1.0).astype(np.float16)
    B, A = oracle.svd_factors(W, 0)
    assert B.shape == (8, 0) and A.shape == (0, 32)
    np.testing.assert_array_equal(oracle.residual(W, B, A), W)


def test_planted_component_is_captured():
    # configuration 2 plants 16 equal singular values well above the noise edge
    _, W = wl.config_inputs(2, T=4)
    B, A = oracle.svd_factors(W, 16)
    R = oracle.residual(W, B, A).astype(np.float64)
    G = W.astype(np.float64)
    sv = np.linalg.svd(G, compute_uv=False)
    assert sv[15] > 1.1 * sv[16]
    # the residual's top singular value is the noise edge, not the planted one
    assert np.linalg.svd(R, compute_uv=False)[0] < 0.9 * sv[15]


def test_residual_single_rounding():
    W = wl.gaussian(15, (16, 32), 0.02).astype(np.float16)
    B = wl.gaussian(16, (16, 2), 0.1).astype(np.float32)
    A = wl.gaussian(17, (2, 32), 0.1).astype(np.float32)
    R = oracle.residual(W, B, A)
    exact = W.astype(np.float64) - B.astype(np.float64) @ A.astype(np.float64)
    ulp = np.spacing(np.abs(R)).astype(np.float64)
    assert np.all(np.abs(R.astype(np.float64) - exact) <= 0.5 * ulp)
