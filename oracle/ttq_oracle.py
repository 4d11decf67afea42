"""TTQ oracle: a plain, slow, obviously correct CPU statement of what the
TTQ q_proj hot path computes.

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product (the HIP library and its
Python binding) never calls it, and it shares no code with the product: no
kernels, headers, helpers, tables or constant generators.

Sources (the pages about arXiv 2603.19296, "TTQ: Activation-Aware Test-Time
Quantization to Accelerate LLM Inference On The Fly", Koike-Akino, Liu, Wang):
  [pd]  paper-daily.com deep reading, §2 (method details), §5, §6
  [nb]  nubint.ai review, section on the proposed method
  [gde] gist.science (German), technical summary §2 (Methodik)
  [gfr] gist.science (French), technical summary §2 A/B (Méthodologie)
  [tl]  thelatestinai.com listing, Tables 14-15 (layer shapes)

Where the pages leave a step open, the reading taken here is stated in the
function that implements it.

Precision.  Statistics and the projection are computed in fp64.  The
quantiser decides integer codes, so it runs in the precision the kernel
uses, fp32, with every operation rounded once (numpy float32 ops on float32
arrays are IEEE single operations; division and sqrt are correctly rounded;
np.rint is round-half-to-even).

Pins (what ties this code to the pages and to mathematics rather than to
itself) live in tests/test_oracle_*.py; every function here has at least one.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "colstats", "colstats_f64", "svd_factors", "svd_right_basis", "lowrank_refresh", "residual", "quantize", "pack",
    "unpack", "dequant", "linear", "linear_dense", "rtn_reference_levels",
    "tiled_code_index", "tile_codes", "untile_codes", "tile_groups", "untile_groups",
    "SLOT_CODE8", "interleave8", "deinterleave8", "device_codes", "codes_from_device",
]


# ---------------------------------------------------------------------------
# O1  Online activation statistics
# ---------------------------------------------------------------------------
def colstats_f64(X, p: float = 2.0, lam: float = 0.4, alpha: float = 0.5) -> np.ndarray:
    """Diagonal activation statistic in fp64, one value per input channel j.

    [pd] §2 defines the AWQ diagonal as diag[X X^T + lambda I]^alpha, computed
    online from each prompt's own X; [gde] §2 and [gfr] §2A write the diagonal
    as a p-norm of the channel's activations plus lambda, raised to alpha.
    Reading taken (the pages disagree on sum / mean / root): the mean over the
    T tokens of |x_tj|^p, no p-th root, lambda added after the mean, alpha
    applied to the sum:  d_j = (mean_t |x_tj|^p + lambda)^alpha.  With p=2 the
    mean is the diagonal of the autocorrelation E[X X^T] used in [pd] §2, and
    lambda acts as the shrinkage of [nb].

    X is [T][d] (tokens x input channels).  T must be at least 1.
    """
    X64 = np.asarray(X).astype(np.float64)
    if X64.ndim != 2 or X64.shape[0] < 1:
        raise ValueError("X must be [T][d] with T >= 1")
    T = X64.shape[0]
    a = np.abs(X64)
    if p == 2.0:
        powed = a * a
    elif p == 1.0:
        powed = a
    else:
        powed = a ** p
    mean = powed.sum(axis=0) / T
    return (mean + lam) ** alpha


def colstats(X, p: float = 2.0, lam: float = 0.4, alpha: float = 0.5) -> np.ndarray:
    """D as fp32: the fp64 statistic of colstats_f64 rounded once (RNE).
    The quantiser below and the projection consume this fp32 D."""
    return colstats_f64(X, p, lam, alpha).astype(np.float32)


# ---------------------------------------------------------------------------
# O2  Static low-rank factors and the residual to quantise
# ---------------------------------------------------------------------------
def svd_factors(W, r: int):
    """Rank-r factors B [d'][r], A [r][d] from the SVD of W, computed once.

    [pd] §2 and [gfr] §2B: W is split into a quantised residual plus B A, with
    B, A initialised from the SVD of W and kept static ([gde] says PCA; the
    SVD reading is taken).  Reading for the split: the balanced one,
    B = U_r Sigma_r^(1/2), A = Sigma_r^(1/2) V_r^T (any split gives the same
    product B A).  Computed in fp64, stored fp32.
    """
    W64 = np.asarray(W).astype(np.float64)
    d_out, d = W64.shape
    if r == 0:
        return np.zeros((d_out, 0), np.float32), np.zeros((0, d), np.float32)
    U, S, Vt = np.linalg.svd(W64, full_matrices=False)
    root = np.sqrt(S[:r])
    B = U[:, :r] * root[None, :]
    A = root[:, None] * Vt[:r, :]
    return B.astype(np.float32), A.astype(np.float32)


def svd_right_basis(W, r: int) -> np.ndarray:
    """The top-r right singular vectors of W as an orthonormal basis [d][r]
    (fp64): the starting point of the online refresh below, at which it
    reproduces the static factors of svd_factors."""
    W64 = np.asarray(W).astype(np.float64)
    _, _, Vt = np.linalg.svd(W64, full_matrices=False)
    return Vt[:r].T.copy()


def lowrank_refresh(W, D32, V):
    """One online update of the rank-r factors for a prompt with statistic D.

    [pd] §5 (limitations): the low-rank factors are initialised statically,
    and an online PCA could update them at extra cost; [gfr] §2B: B, A stay
    static to save cost, though adapting them online is possible.  The pages
    fix no update rule.  Reading taken: the method weights the quantisation
    error of W by the activation statistic ([pd] §2: the error of W D^(1/2)),
    so the factors track the principal subspace of the activation-weighted
    weight M = W D^(1/2), and "online PCA" is one step of subspace (block
    power) iteration on M^T M per prompt, warm-started from the previous
    right basis V (orthonormal [d][r]):

        P  = M^T (M V)                 (d x r)
        V' = orth(P)                   (QR, R with a positive diagonal)
        B  = M V',   A = V'^T D^(-1/2) (so B A = M V' V'^T D^(-1/2))

    and the residual W - B A is then quantised as usual.  Starting from the
    top-r right singular vectors of W with D = 1 this reproduces the static
    factors' product; repeated steps with a fixed D converge to the top-r
    subspace of M, where |(W - B A) D^(1/2)|_F^2 is the Eckart-Young minimum
    sum_{i > r} sigma_i(M)^2.  All in fp64; returns (V', B, A) as fp64."""
    W64 = np.asarray(W).astype(np.float64)
    sq = np.sqrt(np.asarray(D32).astype(np.float64))
    V64 = np.asarray(V).astype(np.float64)
    M = W64 * sq[None, :]
    P = M.T @ (M @ V64)
    Q, R = np.linalg.qr(P)
    sign = np.where(np.diag(R) < 0, -1.0, 1.0)
    Vn = Q * sign[None, :]
    B = M @ Vn
    A = Vn.T / sq[None, :]
    return Vn, B, A


def residual(W, B, A) -> np.ndarray:
    """W_res = fp16(W - B A), with the subtraction done in fp64 on the given
    (fp32) factors and rounded once to fp16.  [pd] §2: the quantised part is
    the residual of the low-rank factors.  With r = 0, W_res = W."""
    W16 = np.asarray(W, dtype=np.float16)
    B = np.asarray(B, dtype=np.float32)
    A = np.asarray(A, dtype=np.float32)
    if B.shape[1] == 0:
        return W16.copy()
    return (W16.astype(np.float64) - B.astype(np.float64) @ A.astype(np.float64)).astype(np.float16)


# ---------------------------------------------------------------------------
# O3  Activation-scaled group round-to-nearest quantiser
# ---------------------------------------------------------------------------
def quantize(W_res, D32, q: int, g: int):
    """Quantise V = W_res D^(1/2) group-wise with round-to-nearest.

    [pd] §2: RTN quantise-dequantise per group of weights; the AWQ closed form
    quantises W D^(1/2) and unscales by D^(-1/2) ([gde] §2, [gfr] §2A).  [gde]
    names the per-group parameters: a scale S and a zero point Z (asymmetric).

    Readings taken where the pages are silent:
      * a group is g consecutive input channels of one output row (the GEMM
        reduction axis);
      * the range is extended to include zero, mn = min(0, min v),
        mx = max(0, max v), so the zero point is an integer inside [0, N];
      * the scale is (mx - mn)/N in fp32, stored as fp16 rounded upward (the
        smallest positive fp16 not below it), and codes are chosen against the
        stored scale; an all-zero group stores scale 1 and zero 0;
      * z = clamp(rint(-mn/s), 0, N), c = clamp(rint(v/s) + z, 0, N), with IEEE
        division and round-half-to-even.

    Steps per group, all in fp32 with single rounding:
      sq_j = sqrt(D_j);  v = w * sq_j;  mn, mx;  s32 = (mx - mn)/N;
      s16 = up-rounded fp16 of s32;  s = s16;  z;  codes.

    Returns codes uint8 [d'][d], scales fp16 [d'][d/g], zeros fp16 [d'][d/g].
    """
    W16 = np.asarray(W_res, dtype=np.float16)
    D32 = np.asarray(D32, dtype=np.float32)
    d_out, d = W16.shape
    if d % g != 0:
        raise ValueError("d must be a multiple of g")
    N = np.float32(2 ** q - 1)
    zero32 = np.float32(0.0)

    sq = np.sqrt(D32)                                    # fp32, correctly rounded
    v = W16.astype(np.float32) * sq[None, :]             # fp32 product, one rounding
    grp = v.reshape(d_out, d // g, g)
    mn = np.minimum(grp.min(axis=2), zero32)
    mx = np.maximum(grp.max(axis=2), zero32)
    s32 = (mx - mn) / N                                  # fp32 subtract, fp32 divide

    s16 = s32.astype(np.float16)                         # RNE ...
    low = s16.astype(np.float32) < s32                   # ... then step up if below
    s16[low] = np.nextafter(s16[low], np.float16(np.inf))
    s16[s16 == 0] = np.float16(2.0 ** -24)               # smallest positive fp16
    empty = mx == mn                                     # all-zero group
    s16[empty] = np.float16(1.0)
    s = s16.astype(np.float32)

    z = np.clip(np.rint(-mn / s), zero32, N) + zero32    # + 0 stores zero as +0
    z[empty] = zero32
    codes = np.clip(np.rint(grp / s[:, :, None]) + z[:, :, None], zero32, N)
    return codes.astype(np.uint8).reshape(d_out, d), s16, z.astype(np.float16)


def dequant(codes, s16, z16, g: int) -> np.ndarray:
    """The dequantised scaled weight V_hat = (c - z) s, fp64 [d'][d]."""
    c = np.asarray(codes).astype(np.float64)
    d_out, d = c.shape
    s = np.repeat(np.asarray(s16).astype(np.float64), g, axis=1)
    z = np.repeat(np.asarray(z16).astype(np.float64), g, axis=1)
    assert s.shape == (d_out, d)
    return (c - z) * s


def rtn_reference_levels(q: int) -> np.ndarray:
    """The integer code grid 0..2^q-1 (used by the brute-force pin)."""
    return np.arange(2 ** q, dtype=np.int64)


# ---------------------------------------------------------------------------
# O4  Packing
# ---------------------------------------------------------------------------
def pack(codes, q: int) -> np.ndarray:
    """Pack q-bit codes into little-endian 32-bit words.

    The pages give no storage format (they only name a Marlin-style kernel,
    [pd] §5).  Format taken: along each output row, consecutive blocks of 32
    codes; each block is q uint32 words forming one bitstream in which code k
    (0..31) occupies bits [q*k, q*k + q).  Result shape [d'][d/32][q].
    """
    c = np.asarray(codes).astype(np.uint64)
    d_out, d = c.shape
    if d % 32:
        raise ValueError("d must be a multiple of 32")
    if c.size and c.max() >= 2 ** q:
        raise ValueError("code does not fit in q bits")
    blk = c.reshape(d_out, d // 32, 32)
    words = np.zeros((d_out, d // 32, q), dtype=np.uint64)
    for k in range(32):
        bit = q * k
        w, off = divmod(bit, 32)
        words[:, :, w] |= (blk[:, :, k] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + q > 32:
            words[:, :, w + 1] |= blk[:, :, k] >> np.uint64(32 - off)
    return words.astype(np.uint32)


def unpack(words, q: int, d: int) -> np.ndarray:
    """Inverse of pack: [d'][d/32][q] uint32 -> codes uint8 [d'][d]."""
    wd = np.asarray(words).astype(np.uint64)
    d_out = wd.shape[0]
    out = np.zeros((d_out, d // 32, 32), dtype=np.uint64)
    mask = np.uint64(2 ** q - 1)
    for k in range(32):
        bit = q * k
        w, off = divmod(bit, 32)
        val = wd[:, :, w] >> np.uint64(off)
        if off + q > 32:
            val |= wd[:, :, w + 1] << np.uint64(32 - off)
        out[:, :, k] = val & mask
    return out.reshape(d_out, d).astype(np.uint8)


# ---------------------------------------------------------------------------
# O4b  Tiled storage order of the packed codes and of the group parameters
# ---------------------------------------------------------------------------
# The pages fix no storage order.  The library stores the canonical words of
# pack() in a tiled order so that one 64-channel step of 32 output rows is one
# contiguous chunk.  This is a pure permutation of words (no bit changes):
#
#   canonical word (row n, 32-channel block b, word w), 0 <= w < q
#   nt = n // 32, r = n % 32        row tile and row inside it
#   ks = b // 2,  h = b % 2         64-channel step and block inside it
#   pos = 4*(w % 2) + 2*h + w // 2  when q == 4, else q*h + w
#   index = ((nt * (d/64) + ks) * 32 + r) * 2q + pos
#
# For q = 4 the 8 words of one row and step are stored as
# b0w0 b0w2 b1w0 b1w2 b0w1 b0w3 b1w1 b1w3.  Scales and zeros (one value per
# row and group gi) go to index (nt * (d/g) + gi) * 32 + r.

def tiled_code_index(n, b, w, q: int, d: int):
    """Flat tiled index of canonical word (n, b, w); numpy-broadcastable."""
    n = np.asarray(n, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    w = np.asarray(w, dtype=np.int64)
    nt, r = n // 32, n % 32
    ks, h = b // 2, b % 2
    if q == 4:
        pos = 4 * (w % 2) + 2 * h + w // 2
    else:
        pos = q * h + w
    return ((nt * (d // 64) + ks) * 32 + r) * (2 * q) + pos


def tile_codes(words, q: int) -> np.ndarray:
    """Canonical [d'][d/32][q] words -> flat tiled uint32 array."""
    words = np.asarray(words, dtype=np.uint32)
    d_out, nb, qq = words.shape
    if qq != q or d_out % 32 or nb % 2:
        raise ValueError("tiling needs d' % 32 == 0 and d % 64 == 0")
    n, b, w = np.meshgrid(np.arange(d_out), np.arange(nb), np.arange(q), indexing="ij")
    out = np.zeros(words.size, dtype=np.uint32)
    out[tiled_code_index(n, b, w, q, nb * 32)] = words
    return out


def untile_codes(flat, q: int, d_out: int, d: int) -> np.ndarray:
    """Inverse of tile_codes."""
    flat = np.asarray(flat, dtype=np.uint32).reshape(-1)
    n, b, w = np.meshgrid(np.arange(d_out), np.arange(d // 32), np.arange(q), indexing="ij")
    return flat[tiled_code_index(n, b, w, q, d)]


# ---------------------------------------------------------------------------
# O4c  Order of the codes inside every 8 (the library's stored format)
# ---------------------------------------------------------------------------
# Before packing, the library reorders the codes of every 8 consecutive input
# channels of a row so that stored slot m holds code SLOT_CODE8[m]: the even
# channels first, then the odd ones.  A decoder that pairs slot j with slot
# j + 4 (two codes per 32-bit register) then gets the channel pairs
# (2j, 2j + 1), i.e. the natural channel order of the input.  The stored
# words are tile_codes(pack(interleave8(codes))).

SLOT_CODE8 = (0, 2, 4, 6, 1, 3, 5, 7)


def interleave8(codes) -> np.ndarray:
    """[d'][d] codes -> the same codes in stored slot order (d % 8 == 0)."""
    c = np.asarray(codes)
    d_out, d = c.shape
    if d % 8:
        raise ValueError("d must be a multiple of 8")
    return c.reshape(d_out, d // 8, 8)[:, :, list(SLOT_CODE8)].reshape(d_out, d)


def deinterleave8(stored) -> np.ndarray:
    """Inverse of interleave8."""
    st = np.asarray(stored)
    d_out, d = st.shape
    out = np.empty_like(st).reshape(d_out, d // 8, 8)
    out[:, :, list(SLOT_CODE8)] = st.reshape(d_out, d // 8, 8)
    return out.reshape(d_out, d)


def device_codes(codes, q: int) -> np.ndarray:
    """The library's stored code words for [d'][d] codes (flat uint32)."""
    return tile_codes(pack(interleave8(codes), q), q)


def codes_from_device(flat, q: int, d_out: int, d: int) -> np.ndarray:
    """Inverse of device_codes: flat stored words -> codes uint8 [d'][d]."""
    return deinterleave8(unpack(untile_codes(flat, q, d_out, d), q, d))


def tile_groups(vals) -> np.ndarray:
    """[d'][ng] per-group values (scales or zeros) -> flat tiled array."""
    vals = np.asarray(vals)
    d_out, ng = vals.shape
    if d_out % 32:
        raise ValueError("tiling needs d' % 32 == 0")
    n, gi = np.meshgrid(np.arange(d_out), np.arange(ng), indexing="ij")
    out = np.zeros(vals.size, dtype=vals.dtype)
    out[((n // 32) * ng + gi) * 32 + n % 32] = vals
    return out


def untile_groups(flat, d_out: int, ng: int) -> np.ndarray:
    """Inverse of tile_groups."""
    flat = np.asarray(flat).reshape(-1)
    n, gi = np.meshgrid(np.arange(d_out), np.arange(ng), indexing="ij")
    return flat[((n // 32) * ng + gi) * 32 + n % 32]


# ---------------------------------------------------------------------------
# O5  The low-bit projection
# ---------------------------------------------------------------------------
def linear(X, codes, s16, z16, D32, g: int, B=None, A=None) -> np.ndarray:
    """Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X), in fp64.

    [pd] §2: the quantised weight is unscaled by D^(-1/2); with the static
    low-rank factors the layer is W_q + B A ([gfr] §2B).  The D^(-1/2) factor
    is applied to the input (pre-scaling, [pd] §5).  X is [T][d], Y is
    [T][d'].  This is the factored evaluation; linear_dense builds the
    effective weight first.
    """
    X64 = np.asarray(X).astype(np.float64)
    Vh = dequant(codes, s16, z16, g)
    rs = 1.0 / np.sqrt(np.asarray(D32).astype(np.float64))
    Y = (X64 * rs[None, :]) @ Vh.T
    if B is not None and np.asarray(B).shape[1] > 0:
        B64 = np.asarray(B).astype(np.float64)
        A64 = np.asarray(A).astype(np.float64)
        Y = Y + (X64 @ A64.T) @ B64.T
    return Y


def linear_dense(X, codes, s16, z16, D32, g: int, B=None, A=None) -> np.ndarray:
    """The same Y through the explicit effective weight
    W_eff = V_hat D^(-1/2) + B A, then Y = X W_eff^T."""
    Vh = dequant(codes, s16, z16, g)
    rs = 1.0 / np.sqrt(np.asarray(D32).astype(np.float64))
    W_eff = Vh * rs[None, :]
    if B is not None and np.asarray(B).shape[1] > 0:
        W_eff = W_eff + np.asarray(B).astype(np.float64) @ np.asarray(A).astype(np.float64)
    return np.asarray(X).astype(np.float64) @ W_eff.T
