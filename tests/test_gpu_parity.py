"""GPU parity: every kernel, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars: D within 1e-5 relative; codes, scales and zeros bit-exact when the
quantiser is given the oracle's fp32 D (and the same W_res); W_res bit-exact;
Y within 1e-3 relative Frobenius error (fp16 operands, fp32 accumulation).
Sizes span several tiles with ragged tails; the full configurations are
checked on sampled outputs the oracle computes row by row."""
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


@pytest.mark.parametrize("cfg,T", [(2, 2048), (4, 333), (5, 16384), (1, 100)])
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


def _gemm_case(cfg, T, q, g, r, sample_rows=None, pad_ld=0, raw=False):
    w = wl.CONFIGS[cfg]
    X, W = cfg_inputs(cfg, T=T)
    D = oracle.colstats(X, w.p, w.lam, w.alpha)
    B, A = (oracle.svd_factors(W, r) if r and cfg <= 3 else (None, None))
    if r and B is None:
        rng = np.random.default_rng(cfg)
        B = (rng.standard_normal((W.shape[0], r)) * 0.013).astype(np.float32)
        A = (rng.standard_normal((r, W.shape[1])) * 0.018).astype(np.float32)
    Wq = oracle.residual(W, B, A) if r else W
    c, s, z = oracle.quantize(Wq, D, q, g)
    say(f"gemm cfg={cfg} T={T} q={q} g={g} r={r} raw={raw}")
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
    assert Yg.dtype == X.dtype and Yg.shape == (T, W.shape[0])
    rows = np.arange(T) if sample_rows is None else sample_rows
    Y0 = oracle.linear(X[rows], c, s, z, D, g, B, A)
    err = rel_fro(Yg[rows], Y0)
    say(f"  rel_fro={err:.3e}")
    assert np.all(np.isfinite(Yg[rows]))
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
def test_gemm_parity_full_cfg5_sampled(q, r, raw):
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 16383],
                                     np.random.default_rng(3).integers(0, 16384, 59)]))
    _gemm_case(5, 16384, q, 32, r, sample_rows=rows, raw=raw)


# ---------------------------------------------------------------------------
# end to end through the handle API (prepare once, project prefill + decode)
# ---------------------------------------------------------------------------
def _e2e(cfg, q, g, r, T=None, prompt=0, sample_rows=None, alpha=None, decode_T=()):
    w = wl.CONFIGS[cfg]
    alpha = w.alpha if alpha is None else alpha
    X, W = cfg_inputs(cfg, T=T, prompt=prompt)
    T = X.shape[0]
    B = A = None
    if r:
        B, A = oracle.svd_factors(W, r)
    say(f"e2e cfg={cfg} q={q} g={g} r={r} T={T} prompt={prompt} alpha={alpha}")
    layer = ttq.TTQLinear(dev(W), q=q, g=g, alpha=alpha, lam=w.lam, p=w.p, r=r, T_max=T, B=B, A=A)
    Xd = dev(X)
    layer.prepare(Xd)
    Yg = host(layer.linear(Xd))
    D0 = oracle.colstats(X, w.p, w.lam, alpha)
    Dg = host(layer.D)
    assert np.max(np.abs(Dg.astype(np.float64) - D0) / D0) <= D_TOL
    # the fp16 copy of D^(-1/2) is the fp32 one rounded to nearest even
    assert host(layer.dinvsqrt16).tobytes() == host(layer.dinvsqrt).astype(np.float16).tobytes()
    Wq = oracle.residual(W, B, A) if r else W
    c0, s0, z0 = oracle.quantize(Wq, D0, q, g)
    cg = oracle.codes_from_device(host(layer.codes).view(np.uint32), q, W.shape[0], W.shape[1])
    agree = np.mean(cg == c0)
    say(f"  code agreement with the oracle's own D: {agree:.6f}")
    assert agree >= 0.999
    rows = np.arange(T) if sample_rows is None else sample_rows
    Y0 = oracle.linear(X[rows], c0, s0, z0, D0, g, B, A)
    err = rel_fro(Yg[rows], Y0)
    say(f"  prefill rel_fro={err:.3e}")
    assert err <= Y_TOL
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


@pytest.mark.parametrize("prompt", [0, 1, 2, 3])
def test_e2e_cfg4_prompts(prompt):
    rows = np.random.default_rng(prompt).integers(0, 8192, 96)
    _e2e(4, 4, 32, 0, prompt=prompt, sample_rows=rows)


@pytest.mark.parametrize("q", [4, 2])
def test_e2e_cfg5_prefill_and_decode(q):
    rows = np.random.default_rng(9).integers(0, 16384, 64)
    _e2e(5, q, 32, 0, sample_rows=rows, decode_T=(1, 16, 64))


@pytest.mark.parametrize("cfg,g,r", [(3, 32, 0), (2, 64, 16)])
def test_e2e_q5(cfg, g, r):
    _e2e(cfg, 5, g, r, T=2048, decode_T=(1, 16, 64))


@pytest.mark.parametrize("cfg,q,g", [(1, 4, 32), (3, 4, 64), (3, 3, 128), (5, 2, 32), (5, 4, 32),
                                     (1, 5, 64), (5, 5, 32), (3, 4, 16), (5, 5, 16)])
def test_linear_few_tokens_single_launch(cfg, q, g):
    # ttq_linear with T <= 64 and r = 0 pre-scales inside its own kernels (one
    # kernel for T <= 4, split-K + reduction above): the output must equal
    # ttq_prescale + ttq_wlowbit_gemm bit for bit (same arithmetic, same K
    # grouping for d_in <= 5120), for contiguous and strided input rows, and
    # the oracle within the tolerance
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
        assert host(Y1).tobytes() == host(Y2).tobytes(), f"T={Td}: single launch differs from prescale + gemm"
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
