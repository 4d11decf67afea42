"""Host-side checks of the C ABI: the library loads, exports every function
include/ttq.h declares, reports sizes, and rejects bad arguments with the
documented status before enqueuing anything.  No call here reaches a kernel
launch, so these run without a GPU."""
import ctypes
import os
import re

import pytest

from test_activation_aware_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttq.h")

# aligned, non-null stand-ins: validation never dereferences them
P = ctypes.c_void_p(1 << 20)
MIS = ctypes.c_void_p((1 << 20) + 4)


@pytest.fixture(scope="module")
def lib():
    # the host checks need the library itself (hipcc cross-compiles it without
    # a GPU); build it once if nothing is built yet
    if not os.path.exists(_capi.LIB_PATH):
        from test_activation_aware_amd.build import build
        build()
    return _capi.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_capi.SIGNATURES) == names


def test_abi_version_and_status_text(lib):
    assert lib.ttq_abi_version() == _capi.ABI_VERSION == 6
    for s in range(7):
        assert lib.ttq_status_string(s).decode().startswith("TTQ_")
    assert lib.ttq_status_string(99) == b"unknown ttq_status"


def _cfg(d_in=5120, d_out=8192, q=4, g=32, r=0, alpha=0.5, lam=0.4, p=2.0):
    return _capi.ttq_config(d_in, d_out, q, g, r, alpha, lam, p)


def test_query_sizes_cfg5(lib):
    sz = _capi.ttq_sizes()
    assert lib.ttq_query_sizes(ctypes.byref(_cfg()), 16384, ctypes.byref(sz)) == 0
    assert sz.codes_bytes == 8192 * 160 * 4 * 4          # 20.97 MB of 4-bit codes
    assert sz.scales_bytes == sz.zeros_bytes == 8192 * 160 * 2
    assert sz.d_bytes == 5120 * 4
    assert sz.dinvsqrt_bytes == 5120 * 4 + 5120 * 2  # fp32, then the fp16 copy
    assert sz.wres_bytes == 0
    assert sz.workspace_bytes == lib.ttq_colstats_workspace_bytes(16384, 5120) > 0
    assert sz.linear_workspace_bytes == lib.ttq_linear_workspace_bytes(16384, 5120, 8192, 0) == 16384 * 5120 * 2
    # a few tokens (16 < T <= 64, r = 0): fp32 partials of 8 K splits, when larger than the pre-scaled input
    assert lib.ttq_linear_workspace_bytes(64, 5120, 8192, 0) == 8 * 64 * 8192 * 4
    assert lib.ttq_linear_workspace_bytes(17, 5120, 8192, 0) == 8 * 17 * 8192 * 4
    assert lib.ttq_linear_workspace_bytes(16, 5120, 8192, 0) == (16 * 5120 * 2 + 255) // 256 * 256
    assert lib.ttq_linear_workspace_bytes(4, 5120, 8192, 0) == (4 * 5120 * 2 + 255) // 256 * 256
    assert lib.ttq_linear_workspace_bytes(65, 5120, 8192, 0) == (65 * 5120 * 2 + 255) // 256 * 256
    assert lib.ttq_linear_workspace_bytes(64, 5120, 8192, 16) == 64 * 5120 * 2 + 64 * 16 * 4
    # T_max below 64: the split-K need at T_max
    assert lib.ttq_query_sizes(ctypes.byref(_cfg()), 32, ctypes.byref(sz)) == 0
    assert sz.linear_workspace_bytes == 8 * 32 * 8192 * 4
    assert lib.ttq_query_sizes(ctypes.byref(_cfg(r=16, q=2)), 100, ctypes.byref(sz)) == 0
    assert sz.wres_bytes == 8192 * 5120 * 2
    # pre-scaled input rounded up to 256 bytes, then Z
    assert sz.linear_workspace_bytes == 100 * 5120 * 2 + 100 * 16 * 4
    assert sz.codes_bytes == 8192 * 160 * 2 * 4
    # q = 5: five words per 32 codes
    assert lib.ttq_query_sizes(ctypes.byref(_cfg(q=5)), 16, ctypes.byref(sz)) == 0
    assert sz.codes_bytes == 8192 * 160 * 5 * 4


def test_prefill_workspace_sizes(lib):
    # rank 16, fp16 input, T > 64: the fused statistic's partial rows (16
    # tokens per row below 16384 tokens, 64 from there) then Z
    assert lib.ttq_prefill_workspace_bytes(16384, 5120, 8192, 16, 1) == 256 * 5120 * 4 + 16384 * 16 * 4
    assert lib.ttq_prefill_workspace_bytes(1000, 4096, 4096, 16, 1) == \
        ((63 * 4096 * 4 + 255) // 256) * 256 + 1000 * 16 * 4
    # otherwise what ttq_linear needs
    for T, r, dt in ((16384, 0, 1), (64, 16, 1), (2048, 16, 0), (5, 0, 1)):
        assert lib.ttq_prefill_workspace_bytes(T, 5120, 8192, r, dt) == lib.ttq_linear_workspace_bytes(T, 5120, 8192, r)
    assert lib.ttq_prefill_workspace_bytes(16, 5120, 8192, 0, 7) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=5), _capi.TTQ_OK),
    (dict(q=1), _capi.TTQ_ERR_INVALID_ARG),
    (dict(q=6), _capi.TTQ_ERR_INVALID_ARG),
    (dict(q=8), _capi.TTQ_ERR_INVALID_ARG),
    (dict(g=16), _capi.TTQ_OK),
    (dict(g=8), _capi.TTQ_ERR_UNSUPPORTED),
    (dict(g=48), _capi.TTQ_ERR_INVALID_ARG),
    (dict(r=8), _capi.TTQ_ERR_UNSUPPORTED),
    (dict(r=-1), _capi.TTQ_ERR_INVALID_ARG),
    (dict(d_in=100), _capi.TTQ_ERR_SHAPE),
    (dict(d_in=64, g=128), _capi.TTQ_ERR_SHAPE),
    (dict(d_out=6), _capi.TTQ_ERR_SHAPE),
    (dict(d_out=48), _capi.TTQ_ERR_SHAPE),
    (dict(d_out=0), _capi.TTQ_ERR_SHAPE),
    (dict(d_in=1 << 22), _capi.TTQ_ERR_SHAPE),
    (dict(d_in=(1 << 22) - 64), _capi.TTQ_OK),
    (dict(alpha=-0.1), _capi.TTQ_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), _capi.TTQ_ERR_INVALID_ARG),
    (dict(p=0.0), _capi.TTQ_ERR_INVALID_ARG),
    (dict(lam=0.0), _capi.TTQ_ERR_INVALID_ARG),
    (dict(lam=0.0, alpha=0.0), _capi.TTQ_OK),
])
def test_config_validation(lib, kw, status):
    sz = _capi.ttq_sizes()
    got = lib.ttq_query_sizes(ctypes.byref(_cfg(**kw)), 16, ctypes.byref(sz))
    assert got == status, lib.ttq_last_error()
    if status:
        assert lib.ttq_last_error() != b""


def test_null_and_alignment(lib):
    # quantize_pack: NULL W, misaligned D
    assert lib.ttq_quantize_pack(64, 128, 4, 32, None, P, P, P, P, None) == _capi.TTQ_ERR_NULL
    assert lib.ttq_quantize_pack(40, 128, 4, 32, P, P, P, P, P, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_quantize_pack(64, 128, 4, 32, P, MIS, P, P, P, None) == _capi.TTQ_ERR_ALIGN
    # colstats: odd ldx, T = 0, lambda = 0 with alpha > 0, small workspace
    assert lib.ttq_colstats(P, 1, 4, 128, 130, 2.0, 0.4, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_ALIGN
    assert lib.ttq_colstats(P, 1, 0, 128, 128, 2.0, 0.4, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_colstats(P, 1, 4, 128, 128, 2.0, 0.0, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_INVALID_ARG
    assert lib.ttq_colstats(P, 1, 4, 128, 128, 2.0, 0.4, 0.5, P, P, P, 4, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_colstats(P, 7, 4, 128, 128, 2.0, 0.4, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_INVALID_ARG
    # strides whose row offsets would leave 64 bits (or any device memory)
    assert lib.ttq_colstats(P, 1, 4, 128, 1 << 62, 2.0, 0.4, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_colstats(P, 0, 3, 128, 1 << 45, 2.0, 0.4, 0.5, P, P, P, 1 << 20, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_prescale(P, 1, 1 << 20, 128, 1 << 40, P, P, None) == _capi.TTQ_ERR_SHAPE
    # gemm: ldy too small, r = 16 without Z, bad output dtype, T = 0 is an accepted no-op
    assert lib.ttq_wlowbit_gemm(8, 128, 64, 4, 32, 0, P, 128, P, P, P, None, None, P, 1, 32, None) \
        == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_wlowbit_gemm(8, 128, 64, 4, 32, 16, P, 128, P, P, P, P, None, P, 1, 64, None) \
        == _capi.TTQ_ERR_NULL
    assert lib.ttq_wlowbit_gemm(8, 128, 64, 4, 32, 0, P, 128, P, P, P, None, None, P, 7, 64, None) \
        == _capi.TTQ_ERR_INVALID_ARG
    assert lib.ttq_wlowbit_gemm(8, 128, 64, 4, 32, 0, P, 120, P, P, P, None, None, P, 1, 64, None) \
        == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_wlowbit_gemm(0, 128, 64, 4, 32, 0, None, 128, None, None, None, None, None,
                                None, 1, 64, None) == _capi.TTQ_OK
    # input strides that a 256-row tile's 32-bit buffer offsets cannot reach
    assert lib.ttq_wlowbit_gemm(300, 128, 64, 4, 32, 0, P, 1 << 22, P, P, P, None, None, P, 1, 64, None) \
        == _capi.TTQ_ERR_SHAPE
    # raw-input gemm: prefill sizes only (T > 64), NULL D^(-1/2), misaligned X, odd ldx
    assert lib.ttq_wlowbit_gemm_raw(64, 128, 64, 4, 32, 0, P, 128, P, P, P, P, None, None, P, 64, None) \
        == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_wlowbit_gemm_raw(65, 128, 64, 4, 32, 0, P, 128, None, P, P, P, None, None, P, 64, None) \
        == _capi.TTQ_ERR_NULL
    assert lib.ttq_wlowbit_gemm_raw(65, 128, 64, 4, 32, 0, MIS, 128, P, P, P, P, None, None, P, 64, None) \
        == _capi.TTQ_ERR_ALIGN
    assert lib.ttq_wlowbit_gemm_raw(65, 128, 64, 4, 32, 0, P, 130, P, P, P, P, None, None, P, 64, None) \
        == _capi.TTQ_ERR_ALIGN
    assert lib.ttq_wlowbit_gemm_raw(65, 128, 64, 4, 32, 16, P, 128, P, P, P, P, P, None, P, 64, None) \
        == _capi.TTQ_ERR_NULL
    assert lib.ttq_wlowbit_gemm_raw(300, 128, 64, 4, 32, 0, P, 1 << 22, P, P, P, P, None, None, P, 64, None) \
        == _capi.TTQ_ERR_SHAPE
    # prescale: d not a multiple of 64, NULL dinvsqrt, misaligned Xs, T = 0 no-op
    assert lib.ttq_prescale(P, 1, 4, 96, 96, P, P, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_prescale(P, 1, 4, 128, 128, None, P, None) == _capi.TTQ_ERR_NULL
    assert lib.ttq_prescale(P, 1, 4, 128, 128, P, MIS, None) == _capi.TTQ_ERR_ALIGN
    assert lib.ttq_prescale(None, 1, 0, 128, 128, None, None, None) == _capi.TTQ_OK
    # the statistic with the fixed per-GPU scratch refuses channel counts past it
    assert lib.ttq_colstats_noalloc(P, 1, 64, 16384 + 64, 16384 + 64, 2.0, 0.4, 0.5, P, P, None) \
        == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_colstats_noalloc(P, 1, 0, 128, 128, 2.0, 0.4, 0.5, P, P, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_colstats_noalloc(P, 1, 4, 128, 128, 2.0, 0.4, 0.5, None, P, None) == _capi.TTQ_ERR_NULL
    # the online refresh: r = 16 only, d_in a multiple of 128, a workspace
    ws = lib.ttq_lowrank_refresh_workspace_bytes(8192, 5120, 16)
    assert ws > 0 and lib.ttq_lowrank_refresh_workspace_bytes(8192, 5120, 8) == 0
    assert lib.ttq_lowrank_refresh(64, 256, 8, P, P, P, P, P, P, 1 << 30, None) == _capi.TTQ_ERR_UNSUPPORTED
    assert lib.ttq_lowrank_refresh(64, 192, 16, P, P, P, P, P, P, 1 << 30, None) == _capi.TTQ_ERR_SHAPE
    assert lib.ttq_lowrank_refresh(64, 256, 16, P, P, None, P, P, P, 1 << 30, None) == _capi.TTQ_ERR_NULL
    assert lib.ttq_lowrank_refresh(64, 256, 16, P, P, P, P, P, P, 16, None) == _capi.TTQ_ERR_SHAPE
    # residual and lowrank_z are built for r = 16 only
    assert lib.ttq_residual(64, 128, 8, P, P, P, P, None) == _capi.TTQ_ERR_UNSUPPORTED
    assert lib.ttq_lowrank_z(4, 128, 0, P, 1, 128, P, P, None) == _capi.TTQ_ERR_INVALID_ARG
    assert lib.ttq_lowrank_z(0, 128, 16, None, 1, 128, None, None, None) == _capi.TTQ_OK


def _buffers(T_max, r=0, workspace_bytes=1 << 30):
    f = P.value if r else None
    return _capi.ttq_buffers(P.value, P.value, P.value, P.value, P.value, f, f, f, P.value, T_max,
                             workspace_bytes)


def test_handle_lifecycle_errors(lib):
    h = ctypes.c_void_p()
    cfg = _cfg(d_in=128, d_out=64)
    bad = _buffers(16, workspace_bytes=4)
    assert lib.ttq_create(ctypes.byref(cfg), ctypes.byref(bad), ctypes.byref(h)) == _capi.TTQ_ERR_SHAPE
    cfg16 = _cfg(d_in=128, d_out=64, r=16)
    assert lib.ttq_create(ctypes.byref(cfg16), ctypes.byref(_buffers(16)), ctypes.byref(h)) == _capi.TTQ_ERR_NULL
    assert lib.ttq_create(ctypes.byref(cfg), ctypes.byref(_buffers(16)), ctypes.byref(h)) == _capi.TTQ_OK
    try:
        # prepare before the weight is bound, linear before prepare
        assert lib.ttq_prepare(h, P, 1, 4, 128, None) == _capi.TTQ_ERR_INVALID_ARG
        assert lib.ttq_linear(h, P, 1, 4, 128, P, 64, P, 1 << 20, None) == _capi.TTQ_ERR_INVALID_ARG
        # r = 0: binding the weight is pure host work (the handle borrows W)
        assert lib.ttq_set_weight(h, P, None) == _capi.TTQ_OK
        assert lib.ttq_set_weight(h, MIS, None) == _capi.TTQ_ERR_ALIGN
        assert lib.ttq_prepare(h, P, 1, 0, 128, None) == _capi.TTQ_ERR_SHAPE
        assert lib.ttq_prepare(h, P, 1, 17, 128, None) == _capi.TTQ_ERR_SHAPE   # > T_max
        assert lib.ttq_prepare(h, P, 1, 4, 64, None) == _capi.TTQ_ERR_SHAPE     # ldx < d
        assert lib.ttq_prepare(h, None, 1, 4, 128, None) == _capi.TTQ_ERR_NULL
        # prefill: validation before anything is enqueued
        assert lib.ttq_prefill(h, P, 1, 0, 128, P, 64, P, 1 << 30, None) == _capi.TTQ_ERR_SHAPE
        assert lib.ttq_prefill(h, P, 1, 17, 128, P, 64, P, 1 << 30, None) == _capi.TTQ_ERR_SHAPE
        assert lib.ttq_prefill(h, P, 1, 4, 128, P, 64, None, 1 << 30, None) == _capi.TTQ_ERR_NULL
        assert lib.ttq_prefill(h, P, 1, 4, 128, P, 64, P, 4, None) == _capi.TTQ_ERR_SHAPE
        assert lib.ttq_prefill(h, P, 1, 4, 128, MIS, 64, P, 1 << 30, None) == _capi.TTQ_ERR_ALIGN
        # argument checks come before the handle's state: an input stride past
        # what the projection's 32-bit tile offsets reach is a shape error
        assert lib.ttq_linear(h, P, 1, 300, 1 << 22, P, 64, P, 1 << 30, None) == _capi.TTQ_ERR_SHAPE
        assert lib.ttq_linear(h, P, 1, 4, (1 << 22) - 8, P, 64, P, 1 << 30, None) == _capi.TTQ_ERR_INVALID_ARG
    finally:
        lib.ttq_destroy(h)
    lib.ttq_destroy(None)
