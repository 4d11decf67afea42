"""GPU parity: every kernel, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars: D within 1e-5 relative; codes, scales and zeros bit-exact when the
quantiser is given the same fp32 D (the oracle's, or the GPU's own D read
back) and the same W_res; W_res bit-exact; Y within 1e-3 relative Frobenius
error (fp16 operands, fp32 accumulation), and at the Qwen3 shapes also within
1e-3 on every token row and on every 256 x 256 output tile, so one wrong
tile fails.  Sizes span several tiles with ragged tails; the launch forms the
benchmark times (256-token tiles, chosen when the grid has at least 1024 of
them or a multiple of 256) are compared on every output."""
import functools

import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
import test_activation_aware_amd as ttq  # noqa: E402

pytestmark = pytest.mark.gpu

Y_TOL = 1e-3
D_TOL = 1e-5


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ttq.load()
    yield
    torch.cuda.synchronize()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@functools.lru_cache(maxsize=8)
def cfg_inputs(cfg, T=None, d_out=None, prompt=0):
    return wl.config_inputs(cfg, prompt=prompt, T=T, d_out=d_out)


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def check_y(Yg, Y0, tag=""):
    """Y against the oracle: relative Frobenius error over the whole output,
    and the same bound on every token row and every 256 x 256 tile."""
    Yg = np.asarray(Yg, np.float64)
    Y0 = np.asarray(Y0, np.float64)
    assert Yg.shape == Y0.shape
    assert np.all(np.isfinite(Yg)), f"{tag}: non-finite outputs"
    d2 = (Yg - Y0) ** 2
    r2 = Y0 ** 2
    err = float(np.sqrt(d2.sum() / r2.sum()))
    row = np.sqrt(d2.sum(axis=1) / r2.sum(axis=1))
    T, n = Y0.shape
    tt, tn = -(-T // 256), -(-n // 256)
    pad = lambda a: np.pad(a, ((0, tt * 256 - T), (0, tn * 256 - n)))
    tile = np.sqrt(pad(d2).reshape(tt, 256, tn, 256).sum(axis=(1, 3)) /
                   pad(r2).reshape(tt, 256, tn, 256).sum(axis=(1, 3)))
    say(f"  {tag} rel_fro={err:.3e} worst row {row.max():.3e} (t={int(row.argmax())}) "
        f"worst tile {tile.max():.3e} {np.unravel_index(int(tile.argmax()), tile.shape)}")
    assert err <= Y_TOL
    assert row.max() <= Y_TOL, f"{tag}: token row {int(row.argmax())} off by {row.max():.3e}"
    assert tile.max() <= Y_TOL, f"{tag}: tile {np.unravel_index(int(tile.argmax()), tile.shape)} off"
    return err


def check_quant_given_d(layer, Wq, q, g):
    """The handle's codes, scales and zeros are bit-exact with the oracle's
    quantiser given the GPU's own fp32 D and the same W_res."""
    Dg = host(layer.D)
    c0, s0, z0 = oracle.quantize(Wq, Dg, q, g)
    d_out, d = Wq.shape
    assert host(layer.codes).view(np.uint32).reshape(-1).tobytes() == oracle.device_codes(c0, q).tobytes(), \
        "codes differ from oracle.quantize given the GPU's D"
    sg = oracle.untile_groups(host(layer.scales), d_out, d // g)
    zg = oracle.untile_groups(host(layer.zeros), d_out, d // g)
    assert sg.view(np.uint16).tobytes() == s0.view(np.uint16).tobytes(), "scales differ"
    assert zg.view(np.uint16).tobytes() == z0.view(np.uint16).tobytes(), "zeros differ"


def effective_weight16(codes, s16, z16, dinv16, g):
    """The fp16 operand the projection kernels feed the matrix cores for each
    weight: fp16(fp16((c - z) s) * fp16(d_j^(-1/2))), each product of two
    fp16 values rounded once to nearest even (numpy forms the product of two
    float16 values exactly in float32 and rounds it once to float16).  The
    oracle's projection uses the exact (c - z) s d_j^(-1/2) instead; the two
    roundings are inside the output tolerance."""
    cz = (codes.astype(np.int32) - np.repeat(z16.astype(np.int32), g, axis=1)).astype(np.float16)
    a = cz * np.repeat(s16.astype(np.float16), g, axis=1)
    return a * np.asarray(dinv16, np.float16)[None, :]


def oracle_dinvsqrt(D32):
    return (1.0 / np.sqrt(D32.astype(np.float64))).astype(np.float32)


# ---------------------------------------------------------------------------
# colstats
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,T", [(1, 2048), (1, 333), (2, 2048), (3, 4096), (3, 1), (4, 8192),
                                   (5, 16384), (5, 4097), (5, 31)])
def test_colstats_parity(cfg, T):
    w = wl.CONFIGS[cfg]
    say(f"colstats cfg={cfg} T={T}")
    X, _ = cfg_inputs(cfg, T=T, d_out=8)
    Dg, Rg = ttq.ttq_colstats(dev(X), w.p, w.lam, w.alpha)
    D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
    Dg, Rg = host(Dg), host(Rg)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL
    R0 = 1.0 / np.sqrt(D0.astype(np.float64))
    assert np.max(np.abs(Rg - R0) / R0) <= D_TOL


@pytest.mark.parametrize("p,alpha,lam", [(1.0, 0.5, 0.4), (1.5, 0.6, 0.4), (2.0, 0.0, 0.4),
                                         (2.0, 0.75, 0.4), (2.0, 0.0, 0.0), (3.0, 0.5, 1.0)])
def test_colstats_hyperparameters(p, alpha, lam):
    say(f"colstats p={p} alpha={alpha} lam={lam}")
    X, _ = cfg_inputs(4, T=1000, d_out=8)
    Dg, _ = ttq.ttq_colstats(dev(X), p, lam, alpha)
    Dg = host(Dg)
    D0 = oracle.colstats(X, p, lam, alpha)
    if alpha == 0.0:
        assert np.all(Dg == 1.0)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL


def test_colstats_deterministic_and_strided():
    X, _ = cfg_inputs(3, T=3000, d_out=8)
    Xd = dev(X)
    a = host(ttq.ttq_colstats(Xd)[0])
    b = host(ttq.ttq_colstats(Xd)[0])
    assert a.tobytes() == b.tobytes()
    # a strided view (ldx > d) gives the same statistic
    wide = torch.zeros((X.shape[0], X.shape[1] + 64), dtype=Xd.dtype, device="cuda")
    wide[:, :X.shape[1]] = Xd
    c = host(ttq.ttq_colstats(wide[:, :X.shape[1]])[0])
    assert a.tobytes() == c.tobytes()


# ---------------------------------------------------------------------------
# quantize_pack: bit-exact given the oracle's D
# ---------------------------------------------------------------------------
def _check_quant(W16, D32, q, g, tag):
    say(f"quantize {tag} q={q} g={g} shape={W16.shape}")
    cg, sg, zg = ttq.ttq_quantize_pack(dev(W16), dev(D32), q, g)
    c0, s0, z0 = oracle.quantize(W16, D32, q, g)
    words0 = oracle.device_codes(c0, q)
    cg = host(cg).view(np.uint32).reshape(-1)
    assert cg.shape == words0.shape
    bad = np.flatnonzero(cg != words0)
    assert bad.size == 0, f"{len(bad)} code words differ, first at {bad[:3].tolist()}"
    assert host(sg).view(np.uint16).tobytes() == oracle.tile_groups(s0).view(np.uint16).tobytes(), "scales differ"
    assert host(zg).view(np.uint16).tobytes() == oracle.tile_groups(z0).view(np.uint16).tobytes(), "zeros differ"


@pytest.mark.parametrize("cfg,q,g", [(1, 4, 32), (2, 3, 32), (3, 4, 32), (3, 4, 64), (3, 4, 128),
                                     (4, 4, 32), (5, 4, 32), (5, 2, 32), (2, 5, 32), (3, 5, 64),
                                     (4, 5, 128), (5, 5, 32), (2, 3, 16), (3, 4, 16), (5, 4, 16)])
def test_quantize_pack_bitexact(cfg, q, g):
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg)
    D = oracle.colstats(X[:1024], w.p, w.lam, w.alpha)
    if w.planted_rank:
        B, A = oracle.svd_factors(W, w.planted_rank)
        W = oracle.residual(W, B, A)
    _check_quant(W, D, q, g, f"cfg{cfg}")


@pytest.mark.parametrize("q", [2, 3, 4, 5])
@pytest.mark.parametrize("g", [16, 32, 64, 128])
def test_quantize_pack_edge_cases(q, g):
    rng = np.random.default_rng(100 * q + g)
    d_out, d = 96, 512
    W = rng.standard_normal((d_out, d)) * 0.02
    W[0] = 0.0                                       # all-zero rows / groups
    W[1, :] = np.abs(W[1, :])                        # one-signed positive
    W[2, :] = -np.abs(W[2, :])                       # one-signed negative
    W[3, :] = 0.0123                                 # constant groups
    W[4] = rng.standard_normal(d) * 1e-6             # scales in the fp16 subnormal range
    W[5] = rng.standard_normal(d) * 1e-3
    W[6] = rng.standard_normal(d) * 4.0              # large weights
    W[7, :g] = 0.0
    W[7, 0] = 6.1e-5                                 # lone tiny element
    # exact-tie rows: values on a quarter grid with D = 1 put v/s on half-integers
    for r in range(8, 24):
        vals = rng.integers(-6, 25, size=d) * 0.25
        vals[::g] = -1.5
        vals[1::g] = 6.0
        W[r] = vals
    # zero-point ties: with D = 1, -min/s is a half-integer (q4: s = 0.5,
    # -mn/s = 2.5; q2: s = 2.5, -mn/s = 0.5; q3: s = 0.5, -mn/s = 3.5;
    # q5: s = 0.25, -mn/s = 2.5)
    lo, hi = {3: (-1.75, 1.75), 5: (-0.625, 7.125)}.get(q, (-1.25, 6.25))
    for r in range(24, 40):
        vals = rng.integers(int(lo * 4), int(hi * 4) + 1, size=d) * 0.25
        vals[::g] = lo
        vals[1::g] = hi
        W[r] = vals
    W16 = W.astype(np.float16)
    D = np.exp(rng.standard_normal(d) * 2.0).astype(np.float32)
    D[:] = np.where(np.arange(d) % 3 == 0, 1.0, D)   # exact ones next to wide-range values
    _check_quant(W16, D, q, g, "edge")
    _check_quant(W16, np.ones(d, np.float32), q, g, "edge-D1")
    _check_quant(W16, np.full(d, 4.0, np.float32), q, g, "edge-D4")


def test_quantize_ragged_rows():
    # row counts that leave workgroups with a single tile or a partial set
    X, W = cfg_inputs(3)
    D = oracle.colstats(X[:256], alpha=0.75)
    _check_quant(W[:96], D, 4, 32, "rows96")
    _check_quant(W[:32], D, 3, 128, "rows32")
    # channel counts that leave a partial 128-channel workgroup (64 channels)
    for d in (192, 320, 384, 448):
        _check_quant(np.ascontiguousarray(W[:64, :d]), D[:d], 4, 64 if d % 128 else 128, f"d{d}")
    # step counts (d / 64) that leave the last workgroup of four one-step
    # waves partly empty, for every group size the one-step form takes
    for d, q, g in ((192, 4, 32), (320, 3, 16), (448, 5, 32), (576, 2, 16), (320, 4, 64)):
        _check_quant(np.ascontiguousarray(W[:96, :d]), D[:d], q, g, f"d{d}q{q}g{g}")


# ---------------------------------------------------------------------------
# residual and low-rank Z
# ---------------------------------------------------------------------------
def test_residual_bitexact_cfg2():
    _, W = cfg_inputs(2)
    B, A = oracle.svd_factors(W, 16)
    say("residual cfg2")
    Rg = host(ttq.ttq_residual(dev(W), dev(B), dev(A)))
    R0 = oracle.residual(W, B, A)
    assert Rg.view(np.uint16).tobytes() == R0.view(np.uint16).tobytes()


def test_residual_bitexact_cfg5_shape():
    _, W = cfg_inputs(5, T=8)
    rng = np.random.default_rng(7)
    # factors of SVD scale (sigma_1 of an 8192x5120 N(0, 0.01^2) matrix is about 1.7)
    B = (rng.standard_normal((W.shape[0], 16)) * 0.013).astype(np.float32)
    A = (rng.standard_normal((16, W.shape[1])) * 0.018).astype(np.float32)
    say("residual cfg5 shape")
    Rg = host(ttq.ttq_residual(dev(W), dev(B), dev(A)))
    R0 = oracle.residual(W, B, A)
    assert Rg.view(np.uint16).tobytes() == R0.view(np.uint16).tobytes()


@pytest.mark.parametrize("cfg,T", [(2, 2048), (4, 333), (5, 16384), (1, 100), (5, 8192), (4, 9001)])
def test_lowrank_z(cfg, T):
    X, W = cfg_inputs(cfg, T=T, d_out=64)
    A = (np.random.default_rng(cfg).standard_normal((16, X.shape[1])) * 0.02).astype(np.float32)
    say(f"lowrank_z cfg={cfg} T={T}")
    Zg = host(ttq.ttq_lowrank_z(dev(X), dev(A)))
    Z0 = X.astype(np.float64) @ A.astype(np.float64).T
    assert rel_fro(Zg, Z0) <= 1e-5


# ---------------------------------------------------------------------------
# wlowbit_gemm given the oracle's codes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,T", [(1, 333), (2, 2048), (5, 4097), (3, 1)])
def test_prescale(cfg, T):
    w = wl.CONFIGS[cfg]
    X, _ = cfg_inputs(cfg, T=T, d_out=64)
    D = oracle.colstats(X, w.p, w.lam, w.alpha)
    R = oracle_dinvsqrt(D)
    say(f"prescale cfg={cfg} T={T}")
    Xs = host(ttq.ttq_prescale(dev(X), dev(R)))
    assert Xs.dtype == np.float16 and Xs.shape == X.shape
    ref = X.astype(np.float64) * R.astype(np.float64)[None, :]
    got = Xs.astype(np.float64)
    # one fp32 rounding, then one fp16 rounding (normal range)
    bound = np.abs(ref) * (2.0 ** -11 + 2.0 ** -23) + 2.0 ** -25
    assert np.all(np.abs(got - ref) <= bound)


def _gemm_case(cfg, T, q, g, r, pad_ld=0, raw=False, d_out=None, product_svd=False):
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=T, d_out=d_out)
    D = oracle.colstats(X, w.p, w.lam, w.alpha)
    B = A = None
    if r and product_svd:      # the product's host SVD (pinned in test_svd_host.py)
        B, A = ttq.svd_factors(W, r)
    elif r and cfg <= 3:
        B, A = oracle.svd_factors(W, r)
    elif r:
        rng = np.random.default_rng(cfg)
        B = (rng.standard_normal((W.shape[0], r)) * 0.013).astype(np.float32)
        A = (rng.standard_normal((r, W.shape[1])) * 0.018).astype(np.float32)
    Wq = oracle.residual(W, B, A) if r else W
    c, s, z = oracle.quantize(Wq, D, q, g)
    say(f"gemm cfg={cfg} T={T} d_out={W.shape[0]} q={q} g={g} r={r} raw={raw}")
    Xd = dev(X)
    Zd = ttq.ttq_lowrank_z(Xd, dev(A)) if r else None
    Xs = Xd if raw else ttq.ttq_prescale(Xd, dev(oracle_dinvsqrt(D)))
    if pad_ld:  # the GEMM on a row-strided view of its input
        wide = torch.zeros((T, X.shape[1] + pad_ld), dtype=torch.float16, device="cuda")
        wide[:, :X.shape[1]] = Xs
        Xs = wide[:, :X.shape[1]]
    parts = (dev(oracle.device_codes(c, q)), dev(oracle.tile_groups(s)), dev(oracle.tile_groups(z)), q, g,
             W.shape[0])
    if raw:  # the raw input, fp16(D^(-1/2)) on the weight side
        Yd = ttq.ttq_wlowbit_gemm_raw(Xs, dev(oracle_dinvsqrt(D).astype(np.float16)), *parts,
                                      B=dev(B) if r else None, Z=Zd)
    else:
        Yd = ttq.ttq_wlowbit_gemm(Xs, *parts, B=dev(B) if r else None, Z=Zd, out_dtype=Xd.dtype)
    Yg = host(Yd)
    del Yd, Xd, Xs
    assert Yg.dtype == X.dtype and Yg.shape == (T, W.shape[0])
    Y0 = oracle.linear(X, c, s, z, D, g, B, A)
    if T >= 256 and W.shape[0] >= 256:
        return check_y(Yg, Y0)
    err = rel_fro(Yg, Y0)
    say(f"  rel_fro={err:.3e}")
    assert np.all(np.isfinite(Yg))
    assert err <= Y_TOL
    return err


@pytest.mark.parametrize("cfg,T,q,g,r", [
    (1, 333, 4, 32, 0), (1, 2048, 4, 32, 0),
    (2, 2048, 3, 32, 16), (2, 1, 3, 32, 16), (2, 300, 3, 32, 0),
    (3, 1000, 4, 32, 0), (3, 1000, 4, 64, 0), (3, 1000, 4, 128, 0), (3, 257, 2, 64, 0), (3, 100, 3, 128, 16),
    (4, 777, 4, 32, 0), (4, 513, 4, 32, 16),
    (1, 333, 5, 32, 0), (2, 2048, 5, 32, 16), (3, 1000, 5, 64, 0), (3, 257, 5, 128, 0), (4, 513, 5, 32, 16),
    (1, 2048, 4, 16, 0), (2, 300, 3, 16, 16), (3, 1000, 4, 16, 0), (4, 777, 2, 16, 16),
])
def test_gemm_parity(cfg, T, q, g, r):
    _gemm_case(cfg, T, q, g, r)


@pytest.mark.parametrize("cfg,T,q,g,r", [
    (1, 1, 4, 32, 0), (1, 5, 4, 32, 0), (2, 2, 3, 32, 16), (2, 33, 3, 32, 16),
    (3, 7, 4, 64, 0), (3, 64, 4, 128, 0), (3, 31, 2, 32, 0), (4, 16, 4, 32, 16), (4, 63, 2, 64, 0),
    (5, 1, 4, 32, 0), (5, 64, 4, 32, 16),
    (1, 3, 5, 32, 0), (2, 40, 5, 32, 16), (3, 17, 5, 64, 0), (4, 64, 5, 128, 0), (5, 1, 5, 32, 0),
    (1, 7, 4, 16, 0), (2, 33, 3, 16, 16), (5, 16, 4, 16, 0),
])
def test_decode_parity(cfg, T, q, g, r):
    """T <= 64 on the pre-scaled input takes the decode kernel."""
    _gemm_case(cfg, T, q, g, r)


@pytest.mark.parametrize("cfg,q,g,r", [(5, q, g, 0) for q in (2, 3, 4, 5) for g in (16, 32, 64, 128)] + [
    (5, 4, 32, 16), (5, 3, 128, 16), (5, 5, 16, 16), (2, 3, 32, 16), (1, 4, 32, 0), (1, 5, 128, 0),
    (3, 2, 16, 0), (4, 5, 64, 16), (4, 4, 128, 0), (3, 4, 128, 16),
])
def test_gemv_parity(cfg, q, g, r):
    """T = 1 on the pre-scaled input takes the dot-product form: every code
    width and group size (G = 128 with wave ranges that end inside a group at
    d_in = 5120), the rank-16 term, fp32 output (cfg 1)."""
    _gemm_case(cfg, 1, q, g, r)


@pytest.mark.parametrize("cfg,T,q,g,r", [(5, T, q, g, 0) for q, g in ((2, 32), (3, 64), (4, 16), (4, 128),
                                                                 (5, 32)) for T in (2, 16)] + [
    (5, 9, 4, 32, 16), (5, 16, 3, 128, 16), (1, 16, 4, 32, 0), (1, 2, 5, 64, 0), (3, 11, 2, 16, 0),
    (4, 16, 5, 16, 16),
])
def test_fewtok_parity(cfg, T, q, g, r):
    """2 <= T <= 16 on the pre-scaled input takes the few-token form (fp32
    output at cfg 1; rounds of fewer steps for T = 16 and g = 16)."""
    _gemm_case(cfg, T, q, g, r)


@pytest.mark.parametrize("cfg,q,g,r", [(5, 4, 32, 0), (5, 2, 64, 16), (5, 5, 16, 0), (4, 3, 128, 16),
                                       (2, 4, 32, 16)])
def test_fewtok_linear_raw_input(cfg, q, g, r):
    """ttq_linear on 2 <= T <= 16 fp16 tokens: the few-token form on the raw
    input with D^(-1/2) on the weight side (and Z for r = 16), against the
    oracle with the handle's own D, for contiguous and strided rows."""
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=256)
    B = A = None
    if r:
        B, A = ttq.svd_factors(W, r)
    say(f"few-token raw linear cfg={cfg} q={q} g={g} r={r}")
    layer = ttq.TTQLinear(dev(W), q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=r, T_max=256,
                          B=B, A=A)
    layer.prepare(dev(X))
    Dg = host(layer.D)
    Wq = oracle.residual(W, B, A) if r else W
    c0, s0, z0 = oracle.quantize(Wq, Dg, q, g)
    d = W.shape[1]
    for Td in (2, 3, 7, 8, 15, 16):
        Xn = wl.decode_inputs(cfg, Td, step=Td)
        Xd = dev(Xn)
        Y1 = host(layer.linear(Xd))
        Xp = torch.zeros((Td, d + 64), dtype=Xd.dtype, device=Xd.device)
        Xp[:, :d] = Xd
        assert host(layer.linear(Xp[:, :d])).tobytes() == Y1.tobytes(), f"T={Td}: strided rows differ"
        e = rel_fro(Y1, oracle.linear(Xn, c0, s0, z0, Dg, g, B, A))
        say(f"  T={Td} rel_fro={e:.3e}")
        assert np.all(np.isfinite(Y1)) and e <= Y_TOL
    layer.close()


def test_gemm_parity_strided_input():
    _gemm_case(3, 300, 4, 32, 0, pad_ld=64)
    _gemm_case(3, 40, 4, 32, 0, pad_ld=64)
    _gemm_case(3, 300, 4, 32, 0, pad_ld=64, raw=True)


@pytest.mark.parametrize("cfg,T,q,g,r", [
    (2, 2048, 3, 32, 16), (2, 65, 5, 64, 0), (3, 1000, 4, 64, 0), (3, 257, 2, 128, 0), (3, 100, 3, 128, 16),
    (4, 777, 4, 32, 0), (4, 513, 5, 32, 16), (5, 4097, 4, 32, 0), (3, 300, 4, 16, 0), (4, 513, 5, 16, 16),
])
def test_gemm_raw_parity(cfg, T, q, g, r):
    """The raw-input form (what ttq_linear runs for fp16 input, T > 64)."""
    _gemm_case(cfg, T, q, g, r, raw=True)


@pytest.mark.parametrize("q,r,raw", [(4, 0, False), (2, 0, False), (4, 16, False), (5, 0, False),
                                     (4, 0, True), (4, 16, True), (2, 0, True)])
def test_gemm_parity_full_cfg5(q, r, raw):
    """The Qwen3-32B q_proj prefill (T = 16384), every output compared."""
    _gemm_case(5, 16384, q, 32, r, raw=raw)


# The 256-token instances (chosen when n = d'/256 * ceil(T/256) >= 1024 or n
# is a multiple of 256) on the Qwen3-32B q_proj weight (5120 -> 8192), every
# output compared, at prompts of 32 to 35 token tiles: each code width and
# group size the benchmark
# times, the rank-16 form with the product's host SVD, the pre-scaled input,
# a token-tile count that is not a multiple of the 4-tile XCD band
# (T = 8741: 35 token tiles) and a ragged last channel tile (d' = 8160).
@pytest.mark.parametrize("T,q,g,r,raw,d_out", [
    (8192, 4, 32, 0, True, None), (8741, 4, 32, 0, True, None), (8741, 4, 32, 0, True, 8160),
    (8192, 2, 32, 0, True, None), (8192, 3, 32, 0, True, None), (8192, 5, 32, 0, True, None),
    (8192, 4, 16, 0, True, None), (8192, 4, 64, 0, True, None), (8192, 4, 128, 0, True, None),
    (8192, 4, 32, 16, True, None), (8741, 3, 32, 16, True, None), (8192, 4, 32, 0, False, None),
    (8741, 2, 64, 0, False, 8160),
])
def test_gemm_full_256_token_tiles(T, q, g, r, raw, d_out):
    _gemm_case(5, T, q, g, r, raw=raw, d_out=d_out, product_svd=True)


# ---------------------------------------------------------------------------
# the dense projection on the effective fp16 weight (long prompts)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,T,q,g,r,d_out", [
    (5, 16384, 4, 32, 0, None), (5, 8741, 4, 32, 0, 8160), (5, 4097, 2, 64, 16, None), (5, 300, 3, 32, 0, None),
    (4, 8192, 4, 32, 16, None), (3, 1000, 5, 128, 0, None), (2, 65, 3, 32, 16, None), (1, 1, 4, 16, 0, None),
])
def test_wexp_gemm_parity(cfg, T, q, g, r, d_out):
    """ttq_wexp_gemm on W_hat formed from the oracle's codes: the oracle's Y
    within the tolerance (every row and tile), and the raw-input low-bit
    kernel's Y on the same codes bit for bit (same fp16 operands, same K
    order)."""
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=T, d_out=d_out)
    X = X.astype(np.float16)
    D = oracle.colstats(X, w.p, w.lam, w.alpha)
    B = A = None
    if r:
        B, A = ttq.svd_factors(W, r)
    Wq = oracle.residual(W, B, A) if r else W
    c, s, z = oracle.quantize(Wq, D, q, g)
    dv16 = oracle_dinvsqrt(D).astype(np.float16)
    Wh = effective_weight16(c, s, z, dv16, g)
    say(f"wexp gemm cfg={cfg} T={T} d_out={W.shape[0]} q={q} g={g} r={r}")
    Xd = dev(X)
    Zd = ttq.ttq_lowrank_z(Xd, dev(A)) if r else None
    Yd = ttq.ttq_wexp_gemm(Xd, dev(Wh), B=dev(B) if r else None, Z=Zd)
    Yg = host(Yd)
    if T > 64:
        Yf = host(ttq.ttq_wlowbit_gemm_raw(Xd, dev(dv16), dev(oracle.device_codes(c, q)),
                                           dev(oracle.tile_groups(s)), dev(oracle.tile_groups(z)), q, g,
                                           W.shape[0], B=dev(B) if r else None, Z=Zd))
        assert Yg.tobytes() == Yf.tobytes(), "dense and low-bit projections differ"
    del Yd, Xd
    Y0 = oracle.linear(X, c, s, z, D, g, B, A)
    if T >= 256 and W.shape[0] >= 256:
        check_y(Yg, Y0)
    else:
        assert rel_fro(Yg, Y0) <= Y_TOL


@pytest.mark.parametrize("cfg,T,d,d_out,q,g", [
    (5, 4097, 5056, None, 4, 32),      # 5056 = 39.5 x 128: a 64-channel last column range
    (2, 4097, None, 8192, 3, 64),      # the planted rank-16 weight of the OPT-350M shape, 8192 rows
    (3, 3900, None, 8192, 5, 16),      # q = 5, two groups per 32-channel block, a ragged token tile
])
def test_handle_dense_lowrank(cfg, T, d, d_out, q, g):
    """r = 16 on a long prompt, a handle given room for W_hat: its effective weight is
    fp16(W_hat + B A) with W_hat from its own codes, scales, zeros and fp16
    D^(-1/2) and B A the product of its factors, both prefill and
    prepare + linear project with it alone, and Y is within the tolerance of
    the oracle's Q[(W - B A) D^(1/2)] D^(-1/2) X + B (A X).

    Weight bound, per element: 1/2 ulp of the fp16 result (its one rounding)
    + 2^-17 sum_k |B_nk A_kj| (the fp32 MFMA sum of the three hi / lo
    products, 48 terms, and the dropped lo x lo term) + 2^-24 sum_k (|B_nk| +
    |A_kj|) (the absolute spacing of an fp16 lo part) + 2^-22 |S| (the fp32
    addition)."""
    w = wl.CONFIGS[cfg]
    X, W = wl.config_inputs(cfg, T=T, d=d, d_out=d_out)
    X = X.astype(np.float16)
    assert T >= ttq.ttq_dense_min_tokens(W.shape[0])
    say(f"dense lowrank cfg={cfg} T={T} d={W.shape[1]} d_out={W.shape[0]} q={q} g={g}")
    layer = ttq.TTQLinear(dev(W), q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=16, T_max=T, expand=True)
    assert layer.wexp is not None
    Xd = dev(X)
    Yp = host(layer.prefill(Xd))
    B = host(layer.B).astype(np.float64)
    A = host(layer.A).astype(np.float64)
    d_o, d_i = W.shape
    cg = oracle.codes_from_device(host(layer.codes).view(np.uint32), q, d_o, d_i)
    sg = oracle.untile_groups(host(layer.scales), d_o, d_i // g)
    zg = oracle.untile_groups(host(layer.zeros), d_o, d_i // g)
    S = effective_weight16(cg, sg, zg, host(layer.dinvsqrt16), g).astype(np.float64) + B @ A
    Wg = host(layer.wexp).astype(np.float64)
    ulp = np.spacing(np.abs(Wg).astype(np.float16)).astype(np.float64)
    bound = (0.5 * ulp + 2.0 ** -17 * (np.abs(B) @ np.abs(A)) + 2.0 ** -22 * np.abs(S)
             + 2.0 ** -24 * (np.abs(B).sum(axis=1)[:, None] + np.abs(A).sum(axis=0)[None, :]))
    err = np.abs(Wg - S)
    say(f"  weight: max err / bound {np.max(err / bound):.3f}, "
        f"{np.count_nonzero(Wg != S.astype(np.float16)) / S.size:.2e} differ from fp16(S)")
    assert np.all(err <= bound)
    del S, Wg, ulp, bound, err
    # prepare + linear: the same weight, so the same Y bit for bit
    layer.prepare(Xd)
    Yl = host(layer.linear(Xd))
    assert Yl.tobytes() == Yp.tobytes()
    Bf, Af = host(layer.B), host(layer.A)
    Wq = oracle.residual(W, Bf, Af)
    D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
    c0, s0, z0 = oracle.quantize(Wq, D0, q, g)
    flips = np.count_nonzero(cg != c0)
    Y0 = oracle.linear(X, c0, s0, z0, D0, g, Bf, Af)
    if flips == 0:
        check_y(Yp, Y0, "prefill")
    else:
        assert rel_fro(Yp, Y0) <= Y_TOL
    layer.close()


def test_handle_dense_path():
    """A handle given room for W_hat (opt-in for r = 0): prepare on
    the Qwen3-32B q_proj prompt writes W_hat equal to its definition from the
    handle's own codes, scales, zeros and fp16 D^(-1/2); the projection runs
    the dense GEMM and equals the low-bit kernel on the same codes bit for
    bit; decode calls keep using the codes."""
    w = wl.CONFIGS[5]
    X, W = cfg_inputs(5)
    T = X.shape[0]
    assert T >= ttq.ttq_dense_min_tokens(W.shape[0])
    layer = ttq.TTQLinear(dev(W), q=4, g=32, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T, expand=True)
    assert layer.wexp is not None
    Xd = dev(X)
    layer.prepare(Xd)
    Y = host(layer.linear(Xd))
    cg = oracle.codes_from_device(host(layer.codes).view(np.uint32), 4, W.shape[0], W.shape[1])
    sg = oracle.untile_groups(host(layer.scales), W.shape[0], W.shape[1] // 32)
    zg = oracle.untile_groups(host(layer.zeros), W.shape[0], W.shape[1] // 32)
    Wh = effective_weight16(cg, sg, zg, host(layer.dinvsqrt16), 32)
    assert host(layer.wexp).view(np.uint16).tobytes() == Wh.view(np.uint16).tobytes(), "W_hat differs"
    Yf = host(ttq.ttq_wlowbit_gemm_raw(Xd, layer.dinvsqrt16, layer.codes, layer.scales, layer.zeros, 4, 32,
                                       W.shape[0]))
    assert Y.tobytes() == Yf.tobytes()
    # a shorter prompt in the same handle takes the low-bit kernel, and a
    # projection longer than that prompt does not use a stale W_hat
    Xs = dev(X[:1000])
    layer.prepare(Xs)
    Ys = host(layer.linear(Xs))
    Yl = host(layer.linear(Xd))
    Yr = host(ttq.ttq_wlowbit_gemm_raw(Xd, layer.dinvsqrt16, layer.codes, layer.scales, layer.zeros, 4, 32,
                                       W.shape[0]))
    assert Yl.tobytes() == Yr.tobytes()
    Ysr = host(ttq.ttq_wlowbit_gemm_raw(Xs, layer.dinvsqrt16, layer.codes, layer.scales, layer.zeros, 4, 32,
                                        W.shape[0]))
    assert Ys.tobytes() == Ysr.tobytes()
    layer.close()


# ---------------------------------------------------------------------------
# online refresh of the rank-16 factors
# ---------------------------------------------------------------------------
def _refresh_compare(W, D, V0, Vg, Bg, Ag, tag):
    """GPU refresh result against the oracle's from the same inputs: the
    product B A and the projector V' V'^T within 1e-5, V' orthonormal."""
    Vo, Bo, Ao = oracle.lowrank_refresh(W, D, V0)
    BAo = Bo @ Ao
    BAg = Bg.astype(np.float64) @ Ag.astype(np.float64)
    e_ba = np.linalg.norm(BAg - BAo) / np.linalg.norm(BAo)
    Vg64 = Vg.astype(np.float64)
    e_pr = np.linalg.norm(Vg64 @ (Vg64.T @ Vo) - Vo) / np.sqrt(Vo.shape[1])
    e_on = np.abs(Vg64.T @ Vg64 - np.eye(Vg.shape[1])).max()
    say(f"  {tag}: B A rel {e_ba:.2e}, subspace {e_pr:.2e}, orthonormality {e_on:.2e}")
    assert e_ba <= 1e-5 and e_pr <= 1e-5 and e_on <= 1e-5
    return Vo


@pytest.mark.parametrize("cfg,d_out", [(2, None), (4, None), (5, None), (5, 4096 + 32)])
def test_lowrank_refresh_parity(cfg, d_out):
    """ttq_lowrank_refresh from the SVD basis with two prompts' statistics in
    turn, against oracle.lowrank_refresh from the same inputs; then W_res from
    the GPU's factors bit-exact with the oracle's residual of them."""
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=1024, d_out=d_out)
    X2 = wl.activations(cfg, 1024, w.d, w.x_dtype, w.n_outliers, w.outlier_factor, prompt=1)
    V0 = oracle.svd_right_basis(W, 16).astype(np.float32)
    say(f"refresh cfg={cfg} d_out={W.shape[0]}")
    Vd = dev(V0)
    Wd = dev(W)
    for step, Xp in enumerate((X, X2)):
        D = oracle.colstats(Xp, w.p, w.lam, w.alpha)
        Vin = host(Vd).copy()
        Bd, Ad = ttq.ttq_lowrank_refresh(Wd, dev(D), Vd)
        _refresh_compare(W, D, Vin, host(Vd), host(Bd), host(Ad), f"step {step}")
    Rg = host(ttq.ttq_residual(Wd, Bd, Ad))
    assert Rg.view(np.uint16).tobytes() == oracle.residual(W, host(Bd), host(Ad)).view(np.uint16).tobytes()


@pytest.mark.parametrize("cfg,q,T,expand", [(2, 3, None, False), (5, 2, 8192, False), (5, 4, None, False),
                                             (5, 4, None, True)])
def test_e2e_prepare_refresh(cfg, q, T, expand):
    """A refreshing handle: prepare (statistic, refresh, residual, quantise)
    then the projection.  D within 1e-5; B A within 1e-5 of the oracle's
    refresh from the SVD basis with the oracle's D; W_res bit-exact given the
    GPU's B, A; codes, scales and zeros bit-exact given the GPU's D and W_res;
    Y within 1e-3 of the oracle's own pipeline (its D, refresh, residual,
    codes and projection).  expand: the handle has room for W_hat, so the
    long prompt's projection is the dense GEMM on W_hat + B A with the
    refreshed factors."""
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=T)
    T = X.shape[0]
    say(f"e2e refresh cfg={cfg} q={q} T={T} expand={expand}")
    layer = ttq.TTQLinear(dev(W), q=q, g=32, alpha=w.alpha, lam=w.lam, p=w.p, r=16, T_max=T, refresh=True,
                          expand=expand)
    V0 = host(layer.V).copy()
    Xd = dev(X)
    layer.prepare(Xd)
    Yg = host(layer.linear(Xd))
    D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
    Dg = host(layer.D)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL
    Bg, Ag = host(layer.B), host(layer.A)
    _refresh_compare(W, D0, V0, host(layer.V), Bg, Ag, "refresh")
    Wq = oracle.residual(W, Bg, Ag)
    assert host(layer.wres).view(np.uint16).tobytes() == Wq.view(np.uint16).tobytes(), "W_res differs"
    check_quant_given_d(layer, Wq, q, 32)
    _, Bo, Ao = oracle.lowrank_refresh(W, D0, V0)
    Bo, Ao = Bo.astype(np.float32), Ao.astype(np.float32)
    c0, s0, z0 = oracle.quantize(oracle.residual(W, Bo, Ao), D0, q, 32)
    Y0 = oracle.linear(X, c0, s0, z0, D0, 32, Bo, Ao)
    e = rel_fro(Yg, Y0)
    say(f"  prefill rel_fro={e:.3e}")
    assert np.all(np.isfinite(Yg)) and e <= Y_TOL
    layer.close()


# ---------------------------------------------------------------------------
# end to end through the handle API (prepare once, project prefill + decode)
# ---------------------------------------------------------------------------
def _e2e(cfg, q, g, r, T=None, prompt=0, alpha=None, decode_T=(), prefill=False):
    w = wl.CONFIGS[cfg]
    alpha = w.alpha if alpha is None else alpha
    X, W = cfg_inputs(cfg, T=T, prompt=prompt)
    T = X.shape[0]
    say(f"e2e cfg={cfg} q={q} g={g} r={r} T={T} prompt={prompt} alpha={alpha}")
    # r > 0: the handle takes its static factors from the product's host SVD
    layer = ttq.TTQLinear(dev(W), q=q, g=g, alpha=alpha, lam=w.lam, p=w.p, r=r, T_max=T)
    B = host(layer.B) if r else None
    A = host(layer.A) if r else None
    Xd = dev(X)
    if prefill:   # ttq_prefill: the statistic (and Z for r = 16) from one read of X
        Yg = host(layer.prefill(Xd))
    else:
        layer.prepare(Xd)
        Yg = host(layer.linear(Xd))
    D0 = oracle.colstats(X, w.p, w.lam, alpha)
    Dg = host(layer.D)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL
    # the fp16 copy of D^(-1/2) is the fp32 one rounded to nearest even
    assert host(layer.dinvsqrt16).tobytes() == host(layer.dinvsqrt).astype(np.float16).tobytes()
    Wq = oracle.residual(W, B, A) if r else W
    if r:
        assert host(layer.wres).view(np.uint16).tobytes() == Wq.view(np.uint16).tobytes(), "W_res differs"
    check_quant_given_d(layer, Wq, q, g)
    c0, s0, z0 = oracle.quantize(Wq, D0, q, g)
    cg = oracle.codes_from_device(host(layer.codes).view(np.uint32), q, W.shape[0], W.shape[1])
    flips = np.flatnonzero(cg != c0)
    say(f"  codes differing from the oracle's own D: {flips.size} of {cg.size}")
    # D agrees to 1e-5, so only codes whose scaled weight sits at a rounding
    # tie of the oracle's quantiser may differ, and then by one level
    assert flips.size <= 1e-4 * cg.size
    assert np.all(np.abs(cg.reshape(-1)[flips].astype(int) - c0.reshape(-1)[flips].astype(int)) == 1)
    Y0 = oracle.linear(X, c0, s0, z0, D0, g, B, A)
    if T >= 256 and W.shape[0] >= 256 and flips.size == 0:
        check_y(Yg, Y0, "prefill")
    else:
        # a flipped code moves a whole output channel by one quantisation step
        # times the input, so only the whole-output bound applies here; the
        # per-row and per-tile bounds are checked with identical codes in the
        # GEMM tests
        e = rel_fro(Yg, Y0)
        say(f"  prefill rel_fro={e:.3e}")
        assert np.all(np.isfinite(Yg)) and e <= Y_TOL
    del Y0, Yg
    for Td in decode_T:
        Xn = wl.decode_inputs(cfg, Td, step=Td)
        Yn = host(layer.linear(dev(Xn)))
        e = rel_fro(Yn, oracle.linear(Xn, c0, s0, z0, D0, g, B, A))
        say(f"  decode T={Td} rel_fro={e:.3e}")
        assert e <= Y_TOL
    layer.close()


def test_e2e_cfg1():
    _e2e(1, 4, 32, 0)


@pytest.mark.parametrize("alpha", [0.5, 0.0])
def test_e2e_cfg2_lowrank(alpha):
    _e2e(2, 3, 32, 16, alpha=alpha)


@pytest.mark.parametrize("g", [16, 32, 64, 128])
def test_e2e_cfg3_groupsize(g):
    _e2e(3, 4, g, 0, T=2048)


@pytest.mark.parametrize("prompt,r", [(0, 0), (1, 0), (2, 0), (3, 0), (0, 16), (3, 16)])
def test_e2e_cfg4_prompts(prompt, r):
    _e2e(4, 4, 32, r, prompt=prompt)


@pytest.mark.parametrize("q,r", [(4, 0), (2, 0), (4, 16), (2, 16)])
def test_e2e_cfg5_prefill_and_decode(q, r):
    _e2e(5, q, 32, r, decode_T=(1, 16, 64))


@pytest.mark.parametrize("cfg,q,g,r,T", [
    (5, 4, 32, 16, None), (5, 2, 32, 16, 16384 + 37), (4, 4, 32, 16, None), (4, 4, 32, 16, 1000),
    (2, 3, 32, 16, None), (2, 3, 32, 16, 65), (2, 3, 32, 16, 40), (5, 4, 32, 0, 8192), (1, 4, 32, 0, None),
])
def test_e2e_prefill(cfg, q, g, r, T):
    """ttq_prefill: prepare and projection of one prompt in one call (the
    statistic and Z fused for r = 16, fp16 input, T > 64)."""
    _e2e(cfg, q, g, r, T=T, prefill=True, decode_T=(1, 16) if cfg >= 2 else ())


@pytest.mark.parametrize("cfg,g,r", [(3, 32, 0), (2, 64, 16)])
def test_e2e_q5(cfg, g, r):
    _e2e(cfg, 5, g, r, T=2048, decode_T=(1, 16, 64))


@pytest.mark.parametrize("cfg,q,g", [(1, 4, 32), (3, 4, 64), (3, 3, 128), (5, 2, 32), (5, 4, 32),
                                     (1, 5, 64), (5, 5, 32), (3, 4, 16), (5, 5, 16)])
def test_linear_few_tokens_single_launch(cfg, q, g):
    # ttq_linear with T <= 64 and r = 0 takes the input as it comes: T = 1,
    # the dot-product form pre-scaling inside (the same bits as ttq_prescale +
    # ttq_wlowbit_gemm); fp16 input with 2 <= T <= 16, the few-token form with
    # D^(-1/2) on the weight side (the prefill GEMM's effective weight: within
    # the tolerance of the pre-scaled form, not bit for bit); fp32 input with
    # 2 <= T <= 16, ttq_prescale + ttq_wlowbit_gemm themselves; 16 < T <= 64,
    # split-K + reduction, equal to ttq_prescale + ttq_wlowbit_gemm bit for
    # bit (same arithmetic, same K grouping for d_in <= 5120).  Contiguous and
    # strided input rows give the same bits, and every form is within the
    # tolerance of the oracle
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=256)
    say(f"few-token linear cfg={cfg} q={q} g={g}")
    layer = ttq.TTQLinear(dev(W), q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=256)
    layer.prepare(dev(X))
    D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
    c0, s0, z0 = oracle.quantize(W, D0, q, g)
    d, d_out = W.shape[1], W.shape[0]
    for Td in (1, 2, 3, 4, 5, 16, 32, 33, 64):
        Xn = wl.decode_inputs(cfg, Td, step=Td)
        Xd = dev(Xn)
        Y1 = layer.linear(Xd)
        Xs = ttq.ttq_prescale(Xd, layer.dinvsqrt)
        Y2 = ttq.ttq_wlowbit_gemm(Xs, layer.codes, layer.scales, layer.zeros, q, g, d_out, out_dtype=Xd.dtype)
        if Td == 1 or Td > 16 or Xd.dtype == torch.float32:
            assert host(Y1).tobytes() == host(Y2).tobytes(), f"T={Td}: single launch differs from prescale + gemm"
        else:
            e12 = rel_fro(host(Y1), host(Y2))
            say(f"  T={Td} weight-side vs pre-scaled input: {e12:.3e}")
            assert e12 <= Y_TOL
        Xp = torch.zeros((Td, d + 64), dtype=Xd.dtype, device=Xd.device)
        Xp[:, :d] = Xd
        Y3 = layer.linear(Xp[:, :d])
        assert host(Y3).tobytes() == host(Y1).tobytes(), f"T={Td}: strided rows differ"
        e = rel_fro(host(Y1), oracle.linear(Xn, c0, s0, z0, D0, g))
        say(f"  T={Td} rel_fro={e:.3e}")
        assert e <= Y_TOL
    layer.close()


def test_long_prompt_past_2gb():
    # a 262144-token prompt (X 2.7 GB, Xs 2.7 GB, Y 4.3 GB: past the 2 GB a
    # 32-bit offset reaches) built by repeating a 4096-token block 64 times;
    # D of the repetition is D of the block (a mean), so the oracle's
    # statistic, codes and projection come from the block alone
    w = wl.CONFIGS[5]
    reps, Tb = 64, 4096
    X, W = cfg_inputs(5, T=Tb)
    T = reps * Tb
    say(f"long prompt T={T} (block of {Tb} x {reps})")
    layer = ttq.TTQLinear(dev(W), q=4, g=32, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T)
    Xd = dev(X).repeat(reps, 1)
    layer.prepare(Xd)
    D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
    Dg = host(layer.D)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL
    c0, s0, z0 = oracle.quantize(W, Dg, 4, 32)          # codes given the GPU's own D: bit-exact
    assert host(layer.codes).view(np.uint32).tobytes() == oracle.device_codes(c0, 4).tobytes()
    Y = layer.linear(Xd)
    rows = np.array([0, 1, 4095, 4096, T // 2 + 7, T - 4097, T - 2, T - 1])
    Yg = host(Y[torch.from_numpy(rows).to(Y.device)])
    del Y, Xd
    c1, s1, z1 = oracle.quantize(W, D0, 4, 32)
    e = rel_fro(Yg, oracle.linear(X[rows % Tb], c1, s1, z1, D0, 32))
    say(f"  sampled rows rel_fro={e:.3e}")
    assert e <= Y_TOL
    # repeated rows give identical outputs
    assert np.array_equal(Yg[0], Yg[3]) and np.array_equal(Yg[2], Yg[5]) and np.array_equal(Yg[2], Yg[7])
    layer.close()


def test_qkv_shared_prepare():
    # q, k and v projections of one input share D: one handle on the stacked
    # weight [Wq; Wk; Wv] (GQA shapes: k, v have fewer rows) prepares once and
    # must give exactly the three separate layers' codes and outputs (prefill,
    # the single-launch and the split-K decode paths)
    w = wl.CONFIGS[3]
    d, T = w.d, 300
    X, Wq = cfg_inputs(3, T=T)
    Wk = wl.weight(3, 512, d, w.w_sigma, part=1)
    Wv = wl.weight(3, 512, d, w.w_sigma, part=2)
    Wqkv = np.concatenate([Wq, Wk, Wv])
    kw = dict(q=4, g=32, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T)
    fused = ttq.TTQLinear(dev(Wqkv), **kw)
    parts = [ttq.TTQLinear(dev(Wi), **kw) for Wi in (Wq, Wk, Wv)]
    Xd = dev(X)
    fused.prepare(Xd)
    for layer in parts:
        layer.prepare(Xd)
    assert host(fused.codes).tobytes() == b"".join(host(layer.codes).tobytes() for layer in parts)
    for Xi in (Xd, dev(wl.decode_inputs(3, 1, step=1)), dev(wl.decode_inputs(3, 16, step=16))):
        Yf = host(fused.linear(Xi))
        Ys = np.concatenate([host(layer.linear(Xi)) for layer in parts], axis=1)
        assert Yf.tobytes() == Ys.tobytes(), f"T={Xi.shape[0]}"
    fused.close()
    for layer in parts:
        layer.close()


def test_alpha_zero_gives_rtn_on_gpu():
    X, W = cfg_inputs(2, T=512)
    layer = ttq.TTQLinear(dev(W), q=3, g=32, alpha=0.0, lam=0.4, r=0, T_max=512)
    layer.prepare(dev(X))
    assert np.all(host(layer.D) == 1.0)
    c0, s0, z0 = oracle.quantize(W, np.ones(W.shape[1], np.float32), 3, 32)
    assert host(layer.codes).view(np.uint32).tobytes() == oracle.device_codes(c0, 3).tobytes()
    assert host(layer.scales).view(np.uint16).tobytes() == oracle.tile_groups(s0).view(np.uint16).tobytes()
    layer.close()


def test_prepare_and_linear_deterministic():
    X, W = cfg_inputs(3, T=1024)
    layer = ttq.TTQLinear(dev(W), q=4, g=32, alpha=0.75, r=0, T_max=1024)
    Xd = dev(X)
    layer.prepare(Xd)
    c1, y1 = host(layer.codes).tobytes(), host(layer.linear(Xd)).tobytes()
    layer.prepare(Xd)
    c2, y2 = host(layer.codes).tobytes(), host(layer.linear(Xd)).tobytes()
    assert c1 == c2 and y1 == y2
    assert host(layer.linear(Xd[:0])).shape == (0, W.shape[0])
    layer.close()
