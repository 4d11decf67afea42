"""ctypes declarations of libttq's C ABI (include/ttq.h).

Loading the library never touches the GPU; only the compute entry points
enqueue work.  A missing library is an error, never a silent fallback."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; TTQ_LIBRARY names another build of the same ABI (for
# example one with sanitizers on its host code)
LIB_PATH = os.environ.get("TTQ_LIBRARY") or os.path.join(PKG, "libttq.so")

TTQ_OK = 0
TTQ_ERR_INVALID_ARG = 1
TTQ_ERR_UNSUPPORTED = 2
TTQ_ERR_SHAPE = 3
TTQ_ERR_NULL = 4
TTQ_ERR_ALIGN = 5
TTQ_ERR_HIP = 6

TTQ_F32 = 0
TTQ_F16 = 1


class ttq_config(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32), ("q", ctypes.c_int32),
                ("g", ctypes.c_int32), ("r", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("lambda_", ctypes.c_float), ("p", ctypes.c_float)]


class ttq_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "codes_bytes", "scales_bytes", "zeros_bytes", "d_bytes", "dinvsqrt_bytes",
        "wres_bytes", "workspace_bytes", "linear_workspace_bytes", "wexp_bytes")]


class ttq_buffers(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("D", ctypes.c_void_p), ("dinvsqrt", ctypes.c_void_p), ("wres", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("A", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("T_max", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("wexp", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t

# name -> (restype, argtypes); every symbol declared in include/ttq.h
SIGNATURES = {
    "ttq_abi_version": (_I32, []),
    "ttq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ttq_last_error": (ctypes.c_char_p, []),
    "ttq_query_sizes": (ctypes.c_int, [ctypes.POINTER(ttq_config), _I64, ctypes.POINTER(ttq_sizes)]),
    "ttq_create": (ctypes.c_int, [ctypes.POINTER(ttq_config), ctypes.POINTER(ttq_buffers),
                                  ctypes.POINTER(_P)]),
    "ttq_destroy": (None, [_P]),
    "ttq_set_weight": (ctypes.c_int, [_P, _P, _P]),
    "ttq_prepare": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P]),
    "ttq_linear_workspace_bytes": (_S, [_I64, _I32, _I32, _I32]),
    "ttq_linear": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P, _I64, _P, _S, _P]),
    "ttq_prefill_workspace_bytes": (_S, [_I64, _I32, _I32, _I32, ctypes.c_int]),
    "ttq_prefill": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P, _I64, _P, _S, _P]),
    "ttq_colstats_workspace_bytes": (_S, [_I64, _I64]),
    "ttq_colstats": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _F, _F, _F, _P, _P, _P, _S, _P]),
    "ttq_colstats_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _F, _F, _F, _P, _P, _P]),
    "ttq_prepare_refresh": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P, _P, _S, _P]),
    "ttq_lowrank_refresh_workspace_bytes": (_S, [_I32, _I32, _I32]),
    "ttq_lowrank_refresh": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _S, _P]),
    "ttq_quantize_pack": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "ttq_residual": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "ttq_lowrank_z": (ctypes.c_int, [_I64, _I32, _I32, _P, ctypes.c_int, _I64, _P, _P, _P]),
    "ttq_prescale": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _I64, _P, _P, _P]),
    "ttq_wlowbit_gemm": (ctypes.c_int, [_I64, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _P, _P,
                                        _P, _P, _P, ctypes.c_int, _I64, _P]),
    "ttq_dense_min_tokens": (_I64, [_I32]),
    "ttq_wexp_gemm": (ctypes.c_int, [_I64, _I32, _I32, _I32, _P, _I64, _P, _P, _P, _P, _I64, _P]),
    "ttq_wlowbit_gemm_raw": (ctypes.c_int, [_I64, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _P, _P,
                                            _P, _P, _P, _P, _I64, _P]),
}

_lib = None


ABI_VERSION = 6  # TTQ_ABI_VERSION of include/ttq.h that these signatures match


def load() -> ctypes.CDLL:
    """The loaded libttq.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m test_activation_aware_amd.build); there is no CPU fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.ttq_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.ttq_abi_version()}, the binding expects "
                               f"{ABI_VERSION}: rebuild the library")
        _lib = lib
    return _lib


class TTQError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        text = lib.ttq_status_string(status).decode()
        detail = lib.ttq_last_error().decode()
        super().__init__(f"{where}: {text} ({detail})")


def check(status: int, where: str) -> None:
    if status != TTQ_OK:
        raise TTQError(status, where)
