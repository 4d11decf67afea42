"""Pins of the oracle's online low-rank refresh (oracle.lowrank_refresh): one
step of subspace iteration on M^T M, M = W D^(1/2), from the previous right
basis.  Each pin ties it to mathematics rather than to itself:
  * fixed point: with D = 1 and the top-r right singular vectors of W (LAPACK),
    B A equals the rank-r truncated SVD of W;
  * convergence to Eckart-Young: repeated steps with a fixed D reach
    sum_{i>r} sigma_i(M)^2 (LAPACK's singular values of M), never increasing
    the residual on the way;
  * the projection identity: (W - B A) D^(1/2) V' = 0 and V'^T V' = I;
  * brute force on a tiny case: P, V', B, A written as explicit loops
    (Gram-Schmidt in place of QR) agree;
  * special cases: r = full rank gives B A = W; a diagonal W with distinct
    weighted entries has the exact answer (the r largest weighted entries)."""
import numpy as np
import pytest

import oracle
import workloads as wl


def _trunc_svd(W64, r):
    U, S, Vt = np.linalg.svd(W64, full_matrices=False)
    return (U[:, :r] * S[:r]) @ Vt[:r]


def test_fixed_point_at_unit_statistic():
    W = wl.weight(2, 256, 192, 0.02, 16, 0.3).astype(np.float64)
    V = oracle.svd_right_basis(W, 16)
    Vn, B, A = oracle.lowrank_refresh(W, np.ones(192, np.float32), V)
    assert np.allclose(B @ A, _trunc_svd(W, 16), atol=1e-12 * np.abs(W).max() * 192)
    # the same subspace
    assert np.allclose(Vn @ Vn.T, V @ V.T, atol=1e-10)


def test_converges_to_eckart_young_of_the_weighted_weight():
    rng = np.random.default_rng(3)
    W = wl.weight(4, 192, 128, 0.015).astype(np.float64)
    D = np.exp(rng.standard_normal(128)).astype(np.float32)
    M = W * np.sqrt(D.astype(np.float64))[None, :]
    sig = np.linalg.svd(M, compute_uv=False)
    optimum = float(np.sum(sig[8:] ** 2))
    V = oracle.svd_right_basis(W, 8)
    prev = np.inf
    for _ in range(400):
        V, B, A = oracle.lowrank_refresh(W, D, V)
        res = float(np.linalg.norm((W - B @ A) * np.sqrt(D.astype(np.float64))[None, :]) ** 2)
        assert res <= prev * (1 + 1e-12)
        prev = res
    assert abs(res - optimum) / optimum <= 1e-8


def test_projection_identity_and_orthonormality():
    rng = np.random.default_rng(5)
    W = wl.weight(3, 160, 96, 0.02).astype(np.float64)
    D = np.exp(rng.standard_normal(96) * 0.8).astype(np.float32)
    V = oracle.svd_right_basis(W, 16)
    Vn, B, A = oracle.lowrank_refresh(W, D, V)
    sq = np.sqrt(D.astype(np.float64))
    assert np.allclose(Vn.T @ Vn, np.eye(16), atol=1e-12)
    assert np.abs(((W - B @ A) * sq[None, :]) @ Vn).max() <= 1e-12 * np.abs(W).max() * 96
    # A undoes the weighting: A D^(1/2) = V'^T
    assert np.allclose(A * sq[None, :], Vn.T, atol=1e-14)


def test_brute_force_tiny():
    rng = np.random.default_rng(7)
    d_out, d, r = 5, 6, 2
    W = rng.standard_normal((d_out, d))
    D = np.exp(rng.standard_normal(d)).astype(np.float32)
    V0, _ = np.linalg.qr(rng.standard_normal((d, r)))
    sq = [float(np.sqrt(np.float64(x))) for x in D]
    M = [[W[n][j] * sq[j] for j in range(d)] for n in range(d_out)]
    MV = [[sum(M[n][j] * V0[j][k] for j in range(d)) for k in range(r)] for n in range(d_out)]
    P = [[sum(M[n][j] * MV[n][k] for n in range(d_out)) for k in range(r)] for j in range(d)]
    # Gram-Schmidt (columns in order) gives Q of the QR with a positive diagonal
    Q = []
    for k in range(r):
        v = [P[j][k] for j in range(d)]
        for q in Q:
            c = sum(v[j] * q[j] for j in range(d))
            v = [v[j] - c * q[j] for j in range(d)]
        nv = sum(x * x for x in v) ** 0.5
        Q.append([x / nv for x in v])
    Vb = np.array(Q).T
    Bb = np.array([[sum(M[n][j] * Vb[j][k] for j in range(d)) for k in range(r)] for n in range(d_out)])
    Ab = np.array([[Vb[j][k] / sq[j] for j in range(d)] for k in range(r)])
    Vn, B, A = oracle.lowrank_refresh(W, D, V0)
    assert np.allclose(Vn, Vb, atol=1e-12) and np.allclose(B, Bb, atol=1e-12) and np.allclose(A, Ab, atol=1e-12)


def test_full_rank_and_diagonal_cases():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((12, 8))
    D = np.exp(rng.standard_normal(8)).astype(np.float32)
    V = oracle.svd_right_basis(W, 8)
    _, B, A = oracle.lowrank_refresh(W, D, V)
    assert np.allclose(B @ A, W, atol=1e-12)
    # diagonal weight: M = diag(w_j sqrt(d_j)); its top-r subspace is the r
    # channels with the largest |w_j| sqrt(d_j), and B A keeps exactly those
    w = np.array([3.0, -1.0, 0.5, 2.0, -0.2, 1.2])   # weighted: 3, 2, 1.5, 1, 0.2, 1.2
    Wd = np.diag(w)
    Dd = np.array([1.0, 4.0, 9.0, 0.25, 1.0, 1.0], np.float32)
    weighted = np.abs(w) * np.sqrt(Dd.astype(np.float64))
    keep = np.argsort(-weighted)[:3]
    V = np.eye(6)[:, keep[[1, 0, 2]]] + 0.01 * rng.standard_normal((6, 3))
    for _ in range(60):
        V, B, A = oracle.lowrank_refresh(Wd, Dd, V)
    expect = np.zeros_like(Wd)
    expect[keep, keep] = w[keep]
    assert np.allclose(B @ A, expect, atol=1e-9)
