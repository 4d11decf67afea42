"""The product's host SVD (test_activation_aware_amd.svd_factors), pinned on
the CPU against LAPACK and the Eckart-Young theorem.

The static rank-r factors B, A are initialised from the SVD of W and kept
fixed (paper-daily.com deep reading, section 2; gist.science French summary,
section 2B).  The product computes them from the Gram matrix of the weight;
these pins use numpy's LAPACK SVD (gesdd), a different routine:
  * Eckart-Young: ||W - B A||_F^2 equals sum_{i>r} sigma_i^2, the smallest
    residual any rank-r product can reach, at the Qwen3-8B (4096 x 4096) and
    Qwen3-32B (8192 x 5120) q_proj shapes;
  * B A equals LAPACK's U_r S_r V_r^T (the subspace itself, not only its
    residual) at the OPT-350M shape with its planted rank-16 component and at
    4096 x 4096 with a flat Gaussian spectrum;
  * the planted rank-16 component of the OPT-350M weight is captured;
  * the balanced split: B^T B = A A^T = diag(sigma_1..r);
  * r = 0 gives empty factors and r > min(d_out, d_in) is rejected."""
import numpy as np
import pytest

import workloads as wl

ttq = pytest.importorskip("test_activation_aware_amd")


def _resid2(W64, B, A):
    return float(np.linalg.norm(W64 - B.astype(np.float64) @ A.astype(np.float64)) ** 2)


@pytest.mark.parametrize("cfg,d_out,d", [(4, 4096, 4096), (5, 8192, 5120)])
def test_eckart_young_at_qwen3_shapes(cfg, d_out, d):
    w = wl.CONFIGS[cfg]
    W64 = wl.weight(cfg, d_out, d, w.w_sigma).astype(np.float64)
    B, A = ttq.svd_factors(W64, 16)
    assert B.shape == (d_out, 16) and A.shape == (16, d) and B.dtype == A.dtype == np.float32
    sig = np.linalg.svd(W64, compute_uv=False)
    optimum = float(np.sum(sig[16:] ** 2))
    got = _resid2(W64, B, A)
    assert abs(got - optimum) / optimum <= 1e-6, (got, optimum)
    # the balanced split: column norms of B and row norms of A are sigma_i
    assert np.allclose(np.sum(B.astype(np.float64) ** 2, axis=0), sig[:16], rtol=1e-5)
    assert np.allclose(np.sum(A.astype(np.float64) ** 2, axis=1), sig[:16], rtol=1e-5)


def _lapack_top(W64, r):
    U, S, Vt = np.linalg.svd(W64, full_matrices=False)
    return (U[:, :r] * S[:r]) @ Vt[:r], S


def test_subspace_matches_lapack_planted_opt350m():
    w = wl.CONFIGS[2]
    W64 = wl.weight(2, w.d_out, w.d, w.w_sigma, w.planted_rank, w.planted_rel_norm).astype(np.float64)
    B, A = ttq.svd_factors(W64, 16)
    ref, S = _lapack_top(W64, 16)
    BA = B.astype(np.float64) @ A.astype(np.float64)
    assert np.linalg.norm(BA - ref) / np.linalg.norm(ref) <= 1e-6
    # the planted component P = c U_p V_p^T (workloads.weight's recipe): the
    # column space of B holds most of U_p (a random 16-dimensional subspace
    # of 1024 dimensions would hold 16/1024 of it)
    rng = np.random.Generator(np.random.PCG64(wl.seed(2, wl.ROLE_PLANTED)))
    Up, _ = np.linalg.qr(rng.standard_normal((w.d_out, 16)))
    Q, _ = np.linalg.qr(B.astype(np.float64))
    captured = np.linalg.norm(Q.T @ Up) ** 2 / 16
    assert captured >= 0.75, captured


def test_subspace_matches_lapack_flat_spectrum_4096():
    # a Gaussian weight's top singular values are nearly equal (sigma_16 /
    # sigma_17 about 1.001 here); the exact factors still equal LAPACK's
    w = wl.CONFIGS[4]
    W64 = wl.weight(4, 4096, 4096, w.w_sigma).astype(np.float64)
    B, A = ttq.svd_factors(W64, 16)
    ref, S = _lapack_top(W64, 16)
    assert S[15] > S[16]
    BA = B.astype(np.float64) @ A.astype(np.float64)
    assert np.linalg.norm(BA - ref) / np.linalg.norm(ref) <= 1e-5


def test_wide_weight_and_edge_ranks():
    W64 = wl.gaussian(11, (96, 160), 0.02)          # d_out < d_in: the other Gram side
    B, A = ttq.svd_factors(W64, 16)
    ref, S = _lapack_top(W64, 16)
    assert np.linalg.norm(B.astype(np.float64) @ A.astype(np.float64) - ref) / np.linalg.norm(ref) <= 1e-6
    # full rank reproduces W
    B, A = ttq.svd_factors(W64, 96)
    assert np.linalg.norm(B.astype(np.float64) @ A.astype(np.float64) - W64) / np.linalg.norm(W64) <= 1e-6
    B, A = ttq.svd_factors(W64, 0)
    assert B.shape == (96, 0) and A.shape == (0, 160)
    with pytest.raises(ValueError):
        ttq.svd_factors(W64, 97)
    # an exactly rank-deficient weight: the missing directions give zero factors
    Wd = np.zeros((64, 64))
    Wd[:8, :8] = np.eye(8)
    B, A = ttq.svd_factors(Wd, 16)
    assert np.all(np.isfinite(B)) and np.all(np.isfinite(A))
    assert np.allclose(B.astype(np.float64) @ A.astype(np.float64), Wd, atol=1e-6)
