"""TTQ (activation-aware test-time quantization) q_proj hot path on MI355X.

Thin Python binding over libttq.so (include/ttq.h).  Every step of the path
runs in the library's HIP kernels; this module only marshals torch tensors
(device memory) and the current HIP stream into the C calls.  There is no CPU
fallback: without the built library, or without a GPU, calls raise.

Functions with the C names take torch tensors:
    ttq_colstats, ttq_quantize_pack, ttq_residual, ttq_lowrank_z,
    ttq_prescale, ttq_wlowbit_gemm, ttq_query_sizes
and TTQLinear wraps the handle API (ttq_create / ttq_set_weight /
ttq_prepare / ttq_linear / ttq_destroy) for one q_proj layer:

    layer = TTQLinear(W, q=4, g=32, alpha=0.5, lam=0.4, p=2.0, r=0, T_max=T)
    layer.prepare(X)        # per prompt: D, codes, scales, zeros
    Y = layer.linear(X)     # prefill projection; later decode batches reuse it

The method: per prompt the channel statistic d_j = (mean_t |x_tj|^p +
lambda)^alpha (paper-daily.com deep reading of arXiv 2603.19296, section 2),
group RTN of (W - B A) D^(1/2), and Y = Q[(W - BA) D^(1/2)] (D^(-1/2) X) +
B (A X) with static factors from the SVD of W (same section; gist.science
French summary, section 2B).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _capi
from ._capi import TTQError, TTQ_F16, TTQ_F32, check, load

__all__ = [
    "TTQError", "TTQLinear", "load", "svd_factors", "ttq_colstats", "ttq_colstats_noalloc", "ttq_quantize_pack",
    "ttq_residual", "ttq_lowrank_z", "ttq_prescale", "ttq_wlowbit_gemm", "ttq_wlowbit_gemm_raw",
    "ttq_query_sizes", "ttq_dense_min_tokens", "ttq_wexp_gemm", "ttq_lowrank_refresh",
    "ttq_colstats_workspace_bytes", "ttq_linear_workspace_bytes", "ttq_abi_version", "code_shape",
    "group_shape",
]


def _torch():
    import torch
    return torch


def _stream() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _dev(t, name: str, dtype=None):
    """Pointer of a device tensor, after checking device, dtype and layout."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _x_args(X, name="X"):
    """(pointer, dtype code, T, ldx) of a row-major [T][>=d] activation."""
    torch = _torch()
    if X.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {X.device})")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if X.dtype == torch.float16:
        dt = TTQ_F16
    elif X.dtype == torch.float32:
        dt = TTQ_F32
    else:
        raise TypeError(f"{name} must be float16 or float32 (got {X.dtype})")
    ld = X.stride(0) if X.shape[0] > 1 else X.shape[1]   # one row: the stride is never used
    return ctypes.c_void_p(X.data_ptr()), dt, X.shape[0], ld


def ttq_abi_version() -> int:
    return load().ttq_abi_version()


def ttq_colstats_workspace_bytes(T: int, d: int) -> int:
    return load().ttq_colstats_workspace_bytes(T, d)


def ttq_linear_workspace_bytes(T: int, d: int, d_out: int, r: int) -> int:
    return load().ttq_linear_workspace_bytes(T, d, d_out, r)


def ttq_query_sizes(d_in, d_out, q, g, r, alpha, lam, p, T_max) -> dict:
    cfg = _capi.ttq_config(d_in, d_out, q, g, r, alpha, lam, p)
    out = _capi.ttq_sizes()
    check(load().ttq_query_sizes(ctypes.byref(cfg), T_max, ctypes.byref(out)), "ttq_query_sizes")
    return {n: getattr(out, n) for n, _ in _capi.ttq_sizes._fields_}


def ttq_colstats(X, p: float = 2.0, lam: float = 0.4, alpha: float = 0.5, D=None, dinvsqrt=None,
                 workspace=None):
    """D, D^(-1/2) (fp32 [d]) of the prompt X [T][d] on the GPU."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    d = X.shape[1]
    D = torch.empty(d, dtype=torch.float32, device=X.device) if D is None else D
    dinvsqrt = torch.empty(d, dtype=torch.float32, device=X.device) if dinvsqrt is None else dinvsqrt
    nbytes = ttq_colstats_workspace_bytes(T, d)
    if workspace is None:
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=X.device)
    check(load().ttq_colstats(x, dt, T, d, ldx, p, lam, alpha, _dev(D, "D", torch.float32),
                              _dev(dinvsqrt, "dinvsqrt", torch.float32),
                              _dev(workspace, "workspace", torch.float32),
                              workspace.numel() * 4, _stream()), "ttq_colstats")
    return D, dinvsqrt


def ttq_colstats_noalloc(X, p: float = 2.0, lam: float = 0.4, alpha: float = 0.5, D=None, dinvsqrt=None):
    """ttq_colstats with the partial sums in the library's fixed per-GPU
    scratch (no workspace; for callers that cannot allocate, d <= 16384)."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    d = X.shape[1]
    D = torch.empty(d, dtype=torch.float32, device=X.device) if D is None else D
    dinvsqrt = torch.empty(d, dtype=torch.float32, device=X.device) if dinvsqrt is None else dinvsqrt
    check(load().ttq_colstats_noalloc(x, dt, T, d, ldx, p, lam, alpha, _dev(D, "D", torch.float32),
                                      _dev(dinvsqrt, "dinvsqrt", torch.float32), _stream()),
          "ttq_colstats_noalloc")
    return D, dinvsqrt


def code_shape(d_out: int, d_in: int, q: int):
    """Shape of the packed codes in the tiled order: [d'/32][d/64][32][2q]."""
    return (d_out // 32, d_in // 64, 32, 2 * q)


def group_shape(d_out: int, d_in: int, g: int):
    """Shape of the scales / zeros in the tiled order: [d'/32][d/g][32]."""
    return (d_out // 32, d_in // g, 32)


def ttq_quantize_pack(W, D, q: int, g: int, codes=None, scales=None, zeros=None):
    """Packed codes (uint32 stored as int32) and fp16 scales, zeros, all in the
    tiled order of include/ttq.h."""
    torch = _torch()
    d_out, d_in = W.shape
    dev = W.device
    codes = torch.empty(code_shape(d_out, d_in, q), dtype=torch.int32, device=dev) if codes is None else codes
    scales = torch.empty(group_shape(d_out, d_in, g), dtype=torch.float16, device=dev) if scales is None else scales
    zeros = torch.empty(group_shape(d_out, d_in, g), dtype=torch.float16, device=dev) if zeros is None else zeros
    check(load().ttq_quantize_pack(d_out, d_in, q, g, _dev(W, "W", torch.float16),
                                   _dev(D, "D", torch.float32), _dev(codes, "codes", torch.int32),
                                   _dev(scales, "scales", torch.float16),
                                   _dev(zeros, "zeros", torch.float16), _stream()),
          "ttq_quantize_pack")
    return codes, scales, zeros


def ttq_residual(W, B, A, out=None):
    """W_res = fp16(W - B A) on the GPU (fp64 sum of the rank-r product)."""
    torch = _torch()
    d_out, d_in = W.shape
    r = B.shape[1]
    out = torch.empty_like(W) if out is None else out
    check(load().ttq_residual(d_out, d_in, r, _dev(W, "W", torch.float16), _dev(B, "B", torch.float32),
                              _dev(A, "A", torch.float32), _dev(out, "W_res", torch.float16), _stream()),
          "ttq_residual")
    return out


def ttq_lowrank_z(X, A, out=None):
    """Z = X A^T, fp32 [T][r]."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    r = A.shape[0]
    out = torch.empty((T, r), dtype=torch.float32, device=X.device) if out is None else out
    check(load().ttq_lowrank_z(T, X.shape[1], r, x, dt, ldx, _dev(A, "A", torch.float32),
                               _dev(out, "Z", torch.float32), _stream()), "ttq_lowrank_z")
    return out


def ttq_prescale(X, dinvsqrt, out=None):
    """Xs = fp16(D^(-1/2) X), [T][d] (the pre-scaled input of ttq_wlowbit_gemm)."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    d = X.shape[1]
    out = torch.empty((T, d), dtype=torch.float16, device=X.device) if out is None else out
    check(load().ttq_prescale(x, dt, T, d, ldx, _dev(dinvsqrt, "dinvsqrt", torch.float32),
                              _dev(out, "Xs", torch.float16), _stream()), "ttq_prescale")
    return out


def ttq_wlowbit_gemm(Xs, codes, scales, zeros, q: int, g: int, d_out: int, B=None, Z=None,
                     out=None, out_dtype=None):
    """Y = V_hat Xs + B Z with the packed codes, from the pre-scaled input of
    ttq_prescale; Y is fp16 unless out / out_dtype say otherwise."""
    torch = _torch()
    xs, dt, T, ldxs = _x_args(Xs, "Xs")
    if dt != TTQ_F16:
        raise TypeError("Xs must be float16 (the output of ttq_prescale)")
    d_in = Xs.shape[1]
    r = 0 if B is None else B.shape[1]
    if out is None:
        out = torch.empty((T, d_out), dtype=out_dtype or torch.float16, device=Xs.device)
    if out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit column stride")
    ydt = {torch.float16: TTQ_F16, torch.float32: TTQ_F32}[out.dtype]
    ldy = out.stride(0) if T > 1 else d_out
    bp = _dev(B, "B", torch.float32) if r else None
    zp = _dev(Z, "Z", torch.float32) if r else None
    check(load().ttq_wlowbit_gemm(T, d_in, d_out, q, g, r, xs, ldxs,
                                  _dev(codes, "codes", torch.int32), _dev(scales, "scales", torch.float16),
                                  _dev(zeros, "zeros", torch.float16), bp, zp,
                                  ctypes.c_void_p(out.data_ptr()), ydt, ldy, _stream()), "ttq_wlowbit_gemm")
    return out


def ttq_wlowbit_gemm_raw(X, dinv16, codes, scales, zeros, q: int, g: int, d_out: int, B=None, Z=None,
                         out=None):
    """Y = (V_hat D^(-1/2)) X + B Z from the raw fp16 input (T > 64), with
    dinv16 the fp16 D^(-1/2) (TTQLinear.dinvsqrt16); Y is fp16."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    if dt != TTQ_F16:
        raise TypeError("X must be float16 for the raw-input GEMM")
    d_in = X.shape[1]
    r = 0 if B is None else B.shape[1]
    if out is None:
        out = torch.empty((T, d_out), dtype=torch.float16, device=X.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.dtype != torch.float16:
        raise ValueError("out must be 2-D fp16 with unit column stride")
    ldy = out.stride(0) if T > 1 else d_out
    bp = _dev(B, "B", torch.float32) if r else None
    zp = _dev(Z, "Z", torch.float32) if r else None
    check(load().ttq_wlowbit_gemm_raw(T, d_in, d_out, q, g, r, x, ldx, _dev(dinv16, "dinv16", torch.float16),
                                      _dev(codes, "codes", torch.int32), _dev(scales, "scales", torch.float16),
                                      _dev(zeros, "zeros", torch.float16), bp, zp,
                                      ctypes.c_void_p(out.data_ptr()), ldy, _stream()), "ttq_wlowbit_gemm_raw")
    return out


def ttq_lowrank_refresh(W, D, V, B=None, A=None, workspace=None):
    """One online step of the rank-16 factors: V (fp32 [d_in][16], updated in
    place) advanced toward the principal subspace of W D^(1/2); returns the
    new B [d_out][16] and A [16][d_in] (fp32)."""
    torch = _torch()
    d_out, d_in = W.shape
    r = V.shape[1]
    dev = W.device
    B = torch.empty((d_out, r), dtype=torch.float32, device=dev) if B is None else B
    A = torch.empty((r, d_in), dtype=torch.float32, device=dev) if A is None else A
    nbytes = load().ttq_lowrank_refresh_workspace_bytes(d_out, d_in, r)
    if workspace is None:
        workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)
    check(load().ttq_lowrank_refresh(d_out, d_in, r, _dev(W, "W", torch.float16), _dev(D, "D", torch.float32),
                                     _dev(V, "V", torch.float32), _dev(B, "B", torch.float32),
                                     _dev(A, "A", torch.float32), ctypes.c_void_p(workspace.data_ptr()),
                                     workspace.numel(), _stream()), "ttq_lowrank_refresh")
    return B, A


def ttq_dense_min_tokens(d_out: int) -> int:
    return load().ttq_dense_min_tokens(d_out)


def ttq_wexp_gemm(X, Wexp, B=None, Z=None, out=None):
    """Y = W_hat X + B Z from an effective fp16 weight W_hat [d_out][d_in]
    (the dense projection of long prompts); Y is fp16."""
    torch = _torch()
    x, dt, T, ldx = _x_args(X)
    if dt != TTQ_F16:
        raise TypeError("X must be float16 for the dense projection")
    d_out, d_in = Wexp.shape
    if X.shape[1] != d_in:
        raise ValueError("X and W_hat disagree on d_in")
    r = 0 if B is None else B.shape[1]
    if out is None:
        out = torch.empty((T, d_out), dtype=torch.float16, device=X.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.dtype != torch.float16:
        raise ValueError("out must be 2-D fp16 with unit column stride")
    ldy = out.stride(0) if T > 1 else d_out
    bp = _dev(B, "B", torch.float32) if r else None
    zp = _dev(Z, "Z", torch.float32) if r else None
    check(load().ttq_wexp_gemm(T, d_in, d_out, r, x, ldx, _dev(Wexp, "Wexp", torch.float16), bp, zp,
                               ctypes.c_void_p(out.data_ptr()), ldy, _stream()), "ttq_wexp_gemm")
    return out


def svd_factors(W, r: int, basis: bool = False):
    """Static rank-r factors B [d'][r], A [r][d] (fp32, balanced split
    B = U_r S_r^(1/2), A = S_r^(1/2) V_r^T) of the top-r SVD of the weight,
    computed once on the host (paper-daily.com deep reading of arXiv
    2603.19296, section 2: factors initialised from the SVD of W and kept
    static; gist.science French summary, section 2B).

    Exact in fp64, not randomised: the r largest eigenpairs of the Gram
    matrix of the weight's narrower side (LAPACK's relatively robust
    representation solver through scipy, asked for those r only), then the
    other side's singular vectors by one product, u_i = W v_i / s_i.  The
    Gram matrix squares the singular values, so the leading ones, the only
    ones used, keep fp64 accuracy.  At the Qwen3-32B q_proj shape
    (8192 x 5120) this takes a few seconds; a randomised range finder with a
    handful of power iterations does not converge there, because the
    spectrum of a Gaussian weight is nearly flat at its top.

    basis=True also returns the orthonormal right basis V [d_in][r] (fp32):
    the starting point of the online refresh (ttq_lowrank_refresh), which
    with a uniform statistic gives back these factors' product."""
    import scipy.linalg

    W64 = np.asarray(W, dtype=np.float64)
    d_out, d_in = W64.shape
    if r == 0:
        empty = (np.zeros((d_out, 0), np.float32), np.zeros((0, d_in), np.float32))
        return empty + (np.zeros((d_in, 0), np.float32),) if basis else empty
    if r < 0 or r > min(d_out, d_in):
        raise ValueError(f"rank r={r} must be in [0, min(d_out, d_in) = {min(d_out, d_in)}]")
    tall = d_out >= d_in
    gram = W64.T @ W64 if tall else W64 @ W64.T
    n = gram.shape[0]
    ev, vecs = scipy.linalg.eigh(gram, subset_by_index=[n - r, n - 1], driver="evr")
    ev, vecs = ev[::-1], vecs[:, ::-1]                     # descending
    S = np.sqrt(np.maximum(ev, 0.0))
    live = S > S[0] * 1e-12 if S[0] > 0 else np.zeros_like(S, dtype=bool)
    inv = np.where(live, 1.0 / np.where(live, S, 1.0), 0.0)
    if tall:
        V = vecs
        U = (W64 @ V) * inv[None, :]
    else:
        U = vecs
        V = (W64.T @ U) * inv[None, :]
    root = np.where(live, np.sqrt(S), 0.0)
    factors = ((U * root[None, :]).astype(np.float32), (root[:, None] * V.T).astype(np.float32))
    return factors + (V.astype(np.float32),) if basis else factors


class TTQLinear:
    """One q_proj through the handle API.  Owns its device buffers (torch);
    the C library only records pointers to them."""

    def __init__(self, W, q: int = 4, g: int = 32, alpha: float = 0.5, lam: float = 0.4,
                 p: float = 2.0, r: int = 0, T_max: int = 16384, B=None, A=None, expand=False,
                 refresh: bool = False):
        """expand: give the handle room for the effective fp16 weight, so that
        prompts of at least ttq_dense_min_tokens(d_out) fp16 tokens run the
        dense projection on it (with r = 16 the weight also carries B A).
        Off by default: the low-bit GEMM on the codes matched or beat the
        dense form in the whole prefill step on all but one of the MI355X
        boxes measured, and needs no d_out x d_in fp16 buffer.
        refresh (r = 16): prepare() refreshes the rank-16 factors online for
        each prompt (ttq_prepare_refresh), starting from the SVD basis."""
        torch = _torch()
        if W.dtype != torch.float16 or W.device.type != "cuda" or not W.is_contiguous():
            raise ValueError("W must be a contiguous fp16 GPU tensor [d_out][d_in]")
        self.d_out, self.d_in = W.shape
        self.q, self.g, self.r = q, g, r
        self.alpha, self.lam, self.p = alpha, lam, p
        self.T_max = T_max
        lib = load()
        self._cfg = _capi.ttq_config(self.d_in, self.d_out, q, g, r, alpha, lam, p)
        sz = _capi.ttq_sizes()
        check(lib.ttq_query_sizes(ctypes.byref(self._cfg), T_max, ctypes.byref(sz)), "ttq_query_sizes")
        dev = W.device
        self.W = W
        self.codes = torch.empty(code_shape(self.d_out, self.d_in, q), dtype=torch.int32, device=dev)
        self.scales = torch.empty(group_shape(self.d_out, self.d_in, g), dtype=torch.float16, device=dev)
        self.zeros = torch.empty(group_shape(self.d_out, self.d_in, g), dtype=torch.float16, device=dev)
        self.D = torch.empty(self.d_in, dtype=torch.float32, device=dev)
        # D^(-1/2): fp32 [d_in], followed by its fp16 copy (sz.dinvsqrt_bytes = 6 d_in)
        self._dinv_buf = torch.empty(sz.dinvsqrt_bytes, dtype=torch.uint8, device=dev)
        self.dinvsqrt = self._dinv_buf[:4 * self.d_in].view(torch.float32)
        self.dinvsqrt16 = self._dinv_buf[4 * self.d_in:6 * self.d_in].view(torch.float16)
        self.workspace = torch.empty(max(1, sz.workspace_bytes // 4), dtype=torch.float32, device=dev)
        self.wexp = torch.empty_like(W) if expand else None
        self.V = self.refresh_workspace = None
        if refresh and r != 16:
            raise ValueError("the online refresh is built for r = 16")
        if r > 0:
            if refresh:
                B, A, V = svd_factors(W.float().cpu().numpy(), r, basis=True)
                self.V = torch.as_tensor(np.ascontiguousarray(V), dtype=torch.float32).to(dev)
                nbytes = lib.ttq_lowrank_refresh_workspace_bytes(self.d_out, self.d_in, r)
                self.refresh_workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)
            elif B is None or A is None:
                B, A = svd_factors(W.float().cpu().numpy(), r)
            self.B = torch.as_tensor(np.ascontiguousarray(B), dtype=torch.float32).to(dev)
            self.A = torch.as_tensor(np.ascontiguousarray(A), dtype=torch.float32).to(dev)
            self.wres = torch.empty_like(W)
        else:
            self.B = self.A = self.wres = None
        # the projection's workspace (pre-scaled input, and Z when r > 0), reused
        # by every call on the current stream and grown on demand
        self.linear_workspace = torch.empty(max(1, sz.linear_workspace_bytes), dtype=torch.uint8, device=dev)
        ptr = lambda t: None if t is None else t.data_ptr()
        self._bufs = _capi.ttq_buffers(ptr(self.codes), ptr(self.scales), ptr(self.zeros), ptr(self.D),
                                       ptr(self.dinvsqrt), ptr(self.wres), ptr(self.B), ptr(self.A),
                                       ptr(self.workspace), T_max, self.workspace.numel() * 4, ptr(self.wexp))
        h = ctypes.c_void_p()
        check(lib.ttq_create(ctypes.byref(self._cfg), ctypes.byref(self._bufs), ctypes.byref(h)), "ttq_create")
        self._h = h
        check(lib.ttq_set_weight(self._h, ctypes.c_void_p(W.data_ptr()), _stream()), "ttq_set_weight")

    def prepare(self, X) -> None:
        """Per-prompt prefill step: D, D^(-1/2), codes, scales and zeros (and,
        for a refreshing layer, the rank-16 factors and W_res first)."""
        x, dt, T, ldx = _x_args(X)
        if X.shape[1] != self.d_in:
            raise ValueError(f"X has {X.shape[1]} channels, the layer {self.d_in}")
        if self.V is not None:
            ws = self.refresh_workspace
            check(load().ttq_prepare_refresh(self._h, x, dt, T, ldx, ctypes.c_void_p(self.V.data_ptr()),
                                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()),
                  "ttq_prepare_refresh")
            return
        check(load().ttq_prepare(self._h, x, dt, T, ldx, _stream()), "ttq_prepare")

    def linear(self, X, out=None):
        """Y [T][d_out] with the current quantisation (prefill or decode)."""
        torch = _torch()
        x, dt, T, ldx = _x_args(X)
        if X.shape[1] != self.d_in:
            raise ValueError(f"X has {X.shape[1]} channels, the layer {self.d_in}")
        out = torch.empty((T, self.d_out), dtype=X.dtype, device=X.device) if out is None else out
        if out.dtype != X.dtype or out.dim() != 2 or out.stride(1) != 1 or out.shape != (T, self.d_out):
            raise ValueError("out must be [T][d_out] with X's dtype and unit column stride")
        ldy = out.stride(0) if T > 1 else self.d_out
        need = ttq_linear_workspace_bytes(T, self.d_in, self.d_out, self.r)
        if self.linear_workspace.numel() < need:
            self.linear_workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        ws = self.linear_workspace
        check(load().ttq_linear(self._h, x, dt, T, ldx, ctypes.c_void_p(out.data_ptr()), ldy,
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()), "ttq_linear")
        return out

    def prefill(self, X, out=None):
        """The whole per-prompt step, prepare(X) then linear(X), in one call
        (ttq_prefill: with r = 16 and fp16 input the statistic and A X come
        from one read of X).  A refreshing layer runs prepare(X) (with the
        refresh) and then linear(X).  Returns Y [T][d_out]."""
        torch = _torch()
        if self.V is not None:
            self.prepare(X)
            return self.linear(X, out=out)
        x, dt, T, ldx = _x_args(X)
        if X.shape[1] != self.d_in:
            raise ValueError(f"X has {X.shape[1]} channels, the layer {self.d_in}")
        out = torch.empty((T, self.d_out), dtype=X.dtype, device=X.device) if out is None else out
        if out.dtype != X.dtype or out.dim() != 2 or out.stride(1) != 1 or out.shape != (T, self.d_out):
            raise ValueError("out must be [T][d_out] with X's dtype and unit column stride")
        ldy = out.stride(0) if T > 1 else self.d_out
        need = load().ttq_prefill_workspace_bytes(T, self.d_in, self.d_out, self.r, dt)
        if self.linear_workspace.numel() < need:
            self.linear_workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        ws = self.linear_workspace
        check(load().ttq_prefill(self._h, x, dt, T, ldx, ctypes.c_void_p(out.data_ptr()), ldy,
                                 ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream()), "ttq_prefill")
        return out

    def close(self) -> None:
        if getattr(self, "_h", None):
            load().ttq_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
