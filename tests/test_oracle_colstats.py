"""Pins for the oracle's activation statistic (colstats).

Each check ties the oracle to the definition on the pages or to mathematics,
not to its own code: hand-worked exact examples, the alpha = 0 reduction, the
mean (not sum) convention via duplication, permutation invariance and an exact
brute force with math.fsum on tiny inputs."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_worked_examples(golden_dir):
    g = _golden(golden_dir, "worked_colstats.json")
    for case in g["cases"]:
        X = np.array(case["X"], dtype=np.float64)
        D = oracle.colstats_f64(X, case["p"], case["lam"], case["alpha"])
        for j, val in case.get("D_exact", {}).items():
            assert D[int(j)] == val, case["name"]
        for j, val in case.get("D_approx", {}).items():
            assert abs(D[int(j)] - val) <= 1e-15 * val, case["name"]


def test_hyperparameters_within_pages(golden_dir):
    h = _golden(golden_dir, "hyperparams.json")
    for w in wl.CONFIGS.values():
        assert h["alpha_min"] <= w.alpha <= h["alpha_max"]
        assert w.lam == h["lambda"] and w.p == h["p"]


def test_alpha_zero_is_identity():
    X = wl.gaussian(1, (37, 64), 3.0)
    for p in (1.0, 2.0, 1.5):
        D = oracle.colstats(X, p=p, lam=0.4, alpha=0.0)
        assert D.dtype == np.float32 and np.all(D == 1.0)


def test_constant_columns_closed_form():
    # a constant column has mean |c|^p whatever T is
    c = np.array([0.0, 1.0, -2.0, 0.125, 7.0])
    for T in (1, 3, 64):
        X = np.tile(c, (T, 1))
        for p, lam, alpha in ((2.0, 0.4, 0.5), (1.0, 0.4, 0.75), (3.0, 1.0, 0.6)):
            D = oracle.colstats_f64(X, p, lam, alpha)
            np.testing.assert_allclose(D, (np.abs(c) ** p + lam) ** alpha, rtol=1e-15)


def test_mean_not_sum_duplication():
    # D([X; X]) = D(X) pins the mean: a sum would double the statistic
    X = wl.gaussian(2, (33, 48), 2.0)
    D1 = oracle.colstats_f64(X, 2.0, 0.4, 0.5)
    D2 = oracle.colstats_f64(np.vstack([X, X]), 2.0, 0.4, 0.5)
    np.testing.assert_allclose(D1, D2, rtol=1e-14)


def test_token_permutation_invariance():
    X = wl.gaussian(3, (41, 32), 1.0)
    perm = np.random.default_rng(0).permutation(41)
    np.testing.assert_allclose(oracle.colstats_f64(X), oracle.colstats_f64(X[perm]), rtol=1e-14)


def test_channel_permutation_equivariance():
    X = wl.gaussian(4, (19, 40), 1.0)
    perm = np.random.default_rng(1).permutation(40)
    np.testing.assert_array_equal(oracle.colstats(X)[perm], oracle.colstats(X[:, perm]))


@pytest.mark.parametrize("p", [1.0, 2.0, 2.5])
def test_bruteforce_fsum(p):
    X = wl.gaussian(5, (7, 5), 4.0)
    lam, alpha = 0.4, 0.6
    D = oracle.colstats_f64(X, p, lam, alpha)
    for j in range(X.shape[1]):
        m = math.fsum(math.pow(abs(float(X[t, j])), p) for t in range(X.shape[0])) / X.shape[0]
        assert abs(D[j] - math.pow(m + lam, alpha)) <= 1e-14 * D[j]


def test_fp32_rounding_is_single_rne():
    X = wl.gaussian(6, (9, 16), 3.0)
    D64 = oracle.colstats_f64(X)
    D32 = oracle.colstats(X)
    # RNE to fp32: the fp32 value is within half an fp32 ulp of the fp64 value
    ulp = np.spacing(D32).astype(np.float64)
    assert np.all(np.abs(D32.astype(np.float64) - D64) <= 0.5 * ulp)


def test_rejects_empty():
    with pytest.raises(ValueError):
        oracle.colstats(np.zeros((0, 8)))


def test_outlier_channels_get_larger_scale():
    # the activation-aware direction: channels with larger activations get larger d_j
    w = wl.CONFIGS[1]
    X, _ = wl.config_inputs(1, T=256)
    s = wl.channel_scales(1, w.d, w.n_outliers, w.outlier_factor)
    D = oracle.colstats(X)
    order = np.argsort(s)
    assert np.corrcoef(np.log(s[order]), np.log(D[order]))[0, 1] > 0.95
