"""Pins for the oracle's activation-scaled group RTN quantiser.

The quantiser is a heuristic plus an encoding, so it is pinned by what the
definition fixes independently of the code: hand-worked groups, brute-force
argmin over the 2^q grid, the half-step error bound, the alpha = 0 and uniform
D reductions, structural invariants of (s, z, c), and the AWQ objective the
pages motivate the method with (activation-weighted error below plain RTN)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_worked_groups(golden_dir):
    for case in _golden(golden_dir, "worked_quantize.json")["cases"]:
        W = np.array(case["W"], dtype=np.float16)
        D = np.array(case["D"], dtype=np.float32)
        c, s, z = oracle.quantize(W, D, case["q"], case["g"])
        assert c.tolist() == case["codes"], case["name"]
        assert s.astype(np.float64).tolist() == case["scales"], case["name"]
        assert z.astype(np.float64).tolist() == case["zeros"], case["name"]
        if "W_hat" in case:
            Wh = oracle.dequant(c, s, z, case["g"]) / np.sqrt(D.astype(np.float64))[None, :]
            assert Wh.tolist() == case["W_hat"]


def _scaled(W, D):
    return W.astype(np.float32) * np.sqrt(D.astype(np.float32))[None, :]


def _bruteforce_check(W, D, q, g):
    c, s, z = oracle.quantize(W, D, q, g)
    v = _scaled(W, D).astype(np.float64)
    d_out, d = W.shape
    N = 2 ** q - 1
    S = np.repeat(s.astype(np.float64), g, axis=1)
    Z = np.repeat(z.astype(np.float64), g, axis=1)
    levels = np.arange(N + 1, dtype=np.float64)
    # distance of every grid point to every element
    err = np.abs(v[:, :, None] - (levels[None, None, :] - Z[:, :, None]) * S[:, :, None])
    best = err.min(axis=2)
    mine = np.abs(v - (c.astype(np.float64) - Z) * S)
    assert np.all(mine <= best + S * 2.0 ** -17), "code is not a nearest grid point"
    return c, s, z, v


def _tiny_groups(seed, q, g, rows=64):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((rows, 4 * g)) * 0.05
    W[0::7, :g] = np.abs(W[0::7, :g])            # one-signed (positive) groups
    W[1::7, g:2 * g] = -np.abs(W[1::7, g:2 * g])  # one-signed (negative) groups
    W[2::7, 2 * g:3 * g] = 0.0                    # all-zero groups
    W[3::7, 3 * g:] = 0.03                        # constant groups
    D = np.exp(rng.standard_normal(4 * g)).astype(np.float32)
    return W.astype(np.float16), D


@pytest.mark.parametrize("q", [2, 3, 4, 5])
@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
def test_bruteforce_argmin_tiny(q, g):
    W, D = _tiny_groups(10 * q + g, q, g)
    _bruteforce_check(W, D, q, g)


@pytest.mark.parametrize("cfg,q,g", [(1, 4, 32), (2, 3, 32), (3, 4, 64), (3, 4, 128), (5, 2, 32)])
def test_bruteforce_argmin_config_slice(cfg, q, g):
    X, W = wl.config_inputs(cfg, T=128, d_out=48)
    D = oracle.colstats(X, 2.0, 0.4, wl.CONFIGS[cfg].alpha)
    _bruteforce_check(W, D, q, g)


@pytest.mark.parametrize("q", [2, 3, 4, 5])
def test_half_step_bound_and_ranges(q):
    g = 32
    X, W = wl.config_inputs(1, T=256, d_out=96)
    D = oracle.colstats(X)
    c, s, z = oracle.quantize(W, D, q, g)
    N = 2 ** q - 1
    v = _scaled(W, D).astype(np.float64)
    S = np.repeat(s.astype(np.float64), g, axis=1)
    Z = np.repeat(z.astype(np.float64), g, axis=1)
    vh = (c.astype(np.float64) - Z) * S
    assert np.all(np.abs(v - vh) <= S * (0.5 + 2.0 ** -17))
    # equivalently on the weight itself, scaled back by D^(-1/2)
    w_err = np.abs(W.astype(np.float64) - vh / np.sqrt(D.astype(np.float64))[None, :])
    assert np.all(w_err <= S / np.sqrt(D.astype(np.float64))[None, :] * (0.5 + 2.0 ** -16))
    assert c.min() >= 0 and c.max() <= N
    zf = z.astype(np.float64)
    assert np.all(zf == np.round(zf)) and zf.min() >= 0 and zf.max() <= N
    # the stored grid covers the zero-inclusive range of every group
    grp = v.reshape(v.shape[0], -1, g)
    rng_ = np.maximum(grp.max(2), 0) - np.minimum(grp.min(2), 0)
    assert np.all(N * s.astype(np.float64) >= rng_ * (1 - 2.0 ** -22))
    # s is the smallest fp16 at or above (mx-mn)/N computed in fp32
    s32 = (np.maximum(grp.max(2), 0) - np.minimum(grp.min(2), 0)).astype(np.float32) / np.float32(N)
    below = np.nextafter(s, np.float16(0)).astype(np.float32)
    assert np.all((below < s32) | (s32 == 0))


def test_alpha_zero_reduces_to_plain_rtn():
    """With alpha = 0, D = 1 exactly, the activation scaling is the identity and
    TTQ is plain group RTN of W.  The RTN below is written per group in plain
    Python over float32 scalars, without the D path."""
    X, W = wl.config_inputs(2, T=64, d_out=16, d=128)
    D = oracle.colstats(X, alpha=0.0)
    assert np.all(D == 1.0)
    q, g = 3, 32
    c, s, z = oracle.quantize(W, D, q, g)
    f32 = np.float32
    N = f32(2 ** q - 1)
    for i in range(W.shape[0]):
        for k in range(W.shape[1] // g):
            grp = [f32(x) for x in W[i, k * g:(k + 1) * g]]
            lo, hi = min(min(grp), f32(0)), max(max(grp), f32(0))
            sc = f32(hi - lo) / N
            sh = np.float16(sc)
            if f32(sh) < sc:
                sh = np.nextafter(sh, np.float16(np.inf))
            sf = f32(sh)
            zp = min(max(np.rint(f32(-lo) / sf), f32(0)), N)
            assert s[i, k] == sh and z[i, k] == zp
            for j, x in enumerate(grp):
                cc = min(max(np.rint(x / sf) + zp, f32(0)), N)
                assert c[i, k * g + j] == cc


def test_uniform_D4_scales_exactly():
    # sqrt(4) = 2 is exact, so codes and zeros match D = 1 and scales double
    _, W = wl.config_inputs(3, T=8, d_out=64)
    one = np.ones(W.shape[1], np.float32)
    c1, s1, z1 = oracle.quantize(W, one, 4, 32)
    c4, s4, z4 = oracle.quantize(W, 4 * one, 4, 32)
    np.testing.assert_array_equal(c1, c4)
    np.testing.assert_array_equal(z1, z4)
    np.testing.assert_array_equal(s1.astype(np.float32) * 2, s4.astype(np.float32))


def test_uniform_D_general_matches_rtn_near_boundaries_only():
    # a uniform D rescales every group by the same factor; only the fp16
    # up-rounding of the scale (relative 2^-11) moves the grid, so the level
    # c - z and the zero point z may differ by one step, and only for values
    # next to a rounding boundary
    _, W = wl.config_inputs(3, T=8, d_out=64)
    one = np.ones(W.shape[1], np.float32)
    c1, s1, z1 = oracle.quantize(W, one, 4, 32)
    c3, _, z3 = oracle.quantize(W, 3 * one, 4, 32)
    Z1 = np.repeat(z1.astype(int), 32, axis=1)
    Z3 = np.repeat(z3.astype(int), 32, axis=1)
    lev = (c1.astype(int) - Z1) - (c3.astype(int) - Z3)
    assert np.abs(lev).max() <= 1
    pos = W.astype(np.float64) / np.repeat(s1.astype(np.float64), 32, axis=1)
    dist = np.abs(pos - np.floor(pos) - 0.5)        # distance to the nearest half-integer
    assert np.all(dist[lev != 0] < 15 * 2.0 ** -10)
    assert np.mean(lev != 0) < 0.01
    # zero points: -mn/s sits next to a half-integer wherever they differ
    W64 = W.astype(np.float64).reshape(64, -1, 32)
    zpos = -np.minimum(W64.min(2), 0) / s1.astype(np.float64)
    zdist = np.abs(zpos - np.floor(zpos) - 0.5)
    assert np.all(zdist[z1 != z3] < 15 * 2.0 ** -10)


@pytest.mark.parametrize("cfg", [1, 4])
def test_activation_weighted_error_below_rtn(cfg):
    """AWQ's objective: the output error ||(W - W_hat) X|| is what the method
    reduces.  On activations with outlier channels, TTQ's scaling must beat
    plain RTN (alpha = 0) on that error; a flipped exponent (scaling by
    D^(-1/2)) makes it worse."""
    w = wl.CONFIGS[cfg]
    X, W = wl.config_inputs(cfg, T=512, d_out=256)
    X64 = X.astype(np.float64)
    errs = {}
    for alpha in (0.0, w.alpha):
        D = oracle.colstats(X, 2.0, 0.4, alpha)
        c, s, z = oracle.quantize(W, D, 4, 32)
        Wh = oracle.dequant(c, s, z, 32) / np.sqrt(D.astype(np.float64))[None, :]
        errs[alpha] = np.linalg.norm(X64 @ (W.astype(np.float64) - Wh).T)
    assert errs[w.alpha] < 0.8 * errs[0.0], errs


def test_zero_point_stored_as_positive_zero():
    W = np.zeros((2, 32), np.float16)
    W[0, :] = np.float16(0.5)       # one-signed positive: z = 0
    W[1, :] = -np.float16(0.0)      # negative zeros: an all-zero group
    c, s, z = oracle.quantize(W, np.ones(32, np.float32), 4, 32)
    assert np.all(z.view(np.uint16) == 0)
