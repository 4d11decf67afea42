"""Seeded synthetic workloads for the TTQ q_proj hot path.

This module only draws random tensors.  It holds none of the method's
arithmetic (no statistics, no quantisation, no projection), so both the CPU
oracle and the HIP path may take their inputs from here.

Shapes follow the architecture tables of the TTQ paper (OPT Table 14, Qwen3
Table 15 on the thelatestinai.com page): a q_proj maps hidden size d to
heads x head_dim = d'.  The pages evaluate on real prompts (WikiText-2, PTB,
C4, ...) with trained weights; neither is available, so heavy-tailed
synthetic activations stand in for them: every input channel j gets a
log-normal scale s_j = exp(N(0,1)), a few seeded channels get an extra
outlier factor, and x_tj = s_j * N(0,1).  Weights are N(0, sigma^2).

Every draw uses numpy's PCG64 with seed
    20260311 + 1000*cfg + 10*role + prompt
and roles X=0, W=1, outlier pick=2, planted component=3, decode X=4.
Values are drawn in fp64 and rounded to nearest-even into the stored dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 20260311
ROLE_X, ROLE_W, ROLE_OUTLIER, ROLE_PLANTED, ROLE_DECODE_X = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One q_proj-shaped configuration."""
    cfg: int
    name: str
    d: int                 # input channels (hidden size)
    d_out: int             # output channels d'
    T: int                 # prefill tokens per prompt
    x_dtype: str           # "f32" or "f16"
    n_outliers: int        # channels given an extra scale factor
    outlier_factor: float
    w_sigma: float
    planted_rank: int      # 0, or rank of the planted low-rank component
    planted_rel_norm: float
    q: tuple               # bit widths exercised
    g: tuple               # group sizes exercised
    alpha: float
    lam: float
    p: float
    r: tuple               # low-rank ranks exercised
    prompts: int = 1
    decode_T: tuple = ()


CONFIGS = {
    1: Workload(1, "opt125m_qproj", 768, 768, 2048, "f32", 8, 20.0, 0.02, 0, 0.0,
                (4,), (32,), 0.5, 0.4, 2.0, (0,)),
    2: Workload(2, "opt350m_qproj", 1024, 1024, 2048, "f16", 8, 20.0, 0.02, 16, 0.3,
                (3,), (32,), 0.5, 0.4, 2.0, (16,)),
    3: Workload(3, "qwen3_1p7b_qproj", 2048, 2048, 4096, "f16", 0, 1.0, 0.02, 0, 0.0,
                (4,), (32, 64, 128), 0.75, 0.4, 2.0, (0,)),
    4: Workload(4, "qwen3_8b_qproj", 4096, 4096, 8192, "f16", 16, 50.0, 0.015, 0, 0.0,
                (4,), (32,), 0.5, 0.4, 2.0, (0, 16), prompts=4),
    5: Workload(5, "qwen3_32b_qproj", 5120, 8192, 16384, "f16", 0, 1.0, 0.01, 0, 0.0,
                (4, 2), (32,), 0.5, 0.4, 2.0, (0, 16), decode_T=(1, 16, 64)),
}


def by_name(name: str) -> Workload:
    """The configuration with the given name (e.g. "qwen3_32b_qproj")."""
    for w in CONFIGS.values():
        if w.name == name:
            return w
    raise KeyError(name)


def seed(cfg: int, role: int, prompt: int = 0) -> int:
    return SEED_BASE + 1000 * cfg + 10 * role + prompt


def _rng(cfg: int, role: int, prompt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed(cfg, role, prompt)))


def _np_dtype(name: str):
    return {"f32": np.float32, "f16": np.float16}[name]


def channel_scales(cfg: int, d: int, n_outliers: int, factor: float,
                   prompt: int = 0) -> np.ndarray:
    """Per-channel scales s_j = exp(N(0,1)), with n_outliers seeded channels
    multiplied by `factor`.  fp64, shape [d]."""
    s = np.exp(_rng(cfg, ROLE_X, prompt).standard_normal(d))
    if n_outliers:
        idx = _rng(cfg, ROLE_OUTLIER, prompt).choice(d, n_outliers, replace=False)
        s[idx] *= factor
    return s


def activations(cfg: int, T: int, d: int, dtype: str, n_outliers: int = 0,
                factor: float = 1.0, prompt: int = 0, role: int = ROLE_X,
                chunk_rows: int = 2048) -> np.ndarray:
    """X [T][d] = s_j * N(0,1), drawn row-chunk by row-chunk in fp64 and
    rounded once to `dtype`.  The channel scales are drawn first from the same
    stream, so X for a given (cfg, prompt) is a pure function of T and d."""
    s = channel_scales(cfg, d, n_outliers, factor, prompt)
    rng = _rng(cfg, role, prompt)
    if role == ROLE_X:
        rng.standard_normal(d)          # the scales used these draws
    out = np.empty((T, d), dtype=_np_dtype(dtype))
    for r0 in range(0, T, chunk_rows):
        r1 = min(T, r0 + chunk_rows)
        out[r0:r1] = (rng.standard_normal((r1 - r0, d)) * s[None, :]).astype(out.dtype)
    return out


def weight(cfg: int, d_out: int, d: int, sigma: float, planted_rank: int = 0,
           planted_rel_norm: float = 0.0, part: int = 0) -> np.ndarray:
    """W [d'][d] fp16 = N(0, sigma^2) (+ optional planted rank-k component).
    `part` selects an independent weight of the same layer shape family
    (0 = q_proj, 1 = k_proj, 2 = v_proj: the seed's prompt slot).

    The planted component is P = c * U V^T with U [d'][k], V [d][k] taken as
    the orthonormal Q factors of Gaussian matrices, and c chosen so that
    ||P||_F = planted_rel_norm * ||G||_F, G being the Gaussian part.  All
    its k singular values equal c."""
    G = _rng(cfg, ROLE_W, part).standard_normal((d_out, d)) * sigma
    planted_rank = min(planted_rank, d_out, d)   # tiny test shapes
    if planted_rank:
        rng = _rng(cfg, ROLE_PLANTED)
        U, _ = np.linalg.qr(rng.standard_normal((d_out, planted_rank)))
        V, _ = np.linalg.qr(rng.standard_normal((d, planted_rank)))
        c = planted_rel_norm * np.linalg.norm(G) / np.sqrt(planted_rank)
        G = G + c * (U @ V.T)
    return G.astype(np.float16)


def config_inputs(cfg: int, prompt: int = 0, T: Optional[int] = None,
                  d: Optional[int] = None, d_out: Optional[int] = None):
    """(X, W) of configuration `cfg`; T, d, d_out may be overridden to get a
    smaller tensor with the same recipe (used by the parity tests)."""
    w = CONFIGS[cfg]
    T = w.T if T is None else T
    d = w.d if d is None else d
    d_out = w.d_out if d_out is None else d_out
    X = activations(cfg, T, d, w.x_dtype, w.n_outliers, w.outlier_factor, prompt)
    W = weight(cfg, d_out, d, w.w_sigma, w.planted_rank, w.planted_rel_norm)
    return X, W


def decode_inputs(cfg: int, T: int, step: int = 0) -> np.ndarray:
    """A decode batch of T new tokens (role decode-X), same channel scales as
    prompt 0 of the configuration."""
    w = CONFIGS[cfg]
    s = channel_scales(cfg, w.d, w.n_outliers, w.outlier_factor, 0)
    rng = _rng(cfg, ROLE_DECODE_X, step)
    return (rng.standard_normal((T, w.d)) * s[None, :]).astype(_np_dtype(w.x_dtype))


def gaussian(seed_value: int, shape, scale: float = 1.0, dtype=np.float64) -> np.ndarray:
    """Plain seeded Gaussian tensor for small tests."""
    rng = np.random.Generator(np.random.PCG64(seed_value))
    return (rng.standard_normal(shape) * scale).astype(dtype)
