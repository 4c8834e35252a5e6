"""ctypes view of libwq.so: the C ABI declared in include/wq.h, nothing more."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")

WQ_OK = 0
WQ_ERR_INVALID_ARG = 1
WQ_ERR_UNSUPPORTED = 2
WQ_ERR_MISALIGNED = 3
WQ_ERR_HIP = 4

WQ_PATH_AUTO = 0
WQ_PATH_GEMV = 1
WQ_PATH_MFMA = 2

WQ_SCHEME_ASYM = 0
WQ_SCHEME_SYM = 1
WQ_SCHEME_SYM_TENSOR = 2
WQ_SCHEME_NF4 = 3
WQ_SCHEME_OFFSET = 4

# Every symbol include/wq.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


class GemmItem(ctypes.Structure):
    """wq_gemm_item: the arguments of one wq_gemm call."""
    _fields_ = [("X", _P), ("codes", _P), ("scales", _P), ("zeros", _P), ("Y", _P),
                ("B", _I64), ("K", _I64), ("N", _I64), ("group", _I32), ("bits", _I32)]


class KvCache(ctypes.Structure):
    """wq_kv_cache: the buffers of an int4 KV cache (device pointers)."""
    _fields_ = [("kcodes", _P), ("kscales", _P), ("kzeros", _P), ("vcodes", _P),
                ("vscales", _P), ("vzeros", _P), ("kres", _P), ("vres", _P),
                ("heads", _I64), ("max_blocks", _I64)]


SIGNATURES = {
    "wq_quantize_pack": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _P, _P, _P]),
    "wq_quantize_pack_ex": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "wq_quantize_workspace_size": (ctypes.c_int, [_I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "wq_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P]),
    "wq_gemm_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _SZ, _P]),
    "wq_gemm_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P]),
    "wq_gemm_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "wq_gemm_grouped": (ctypes.c_int, [ctypes.POINTER(GemmItem), _I32, _P, _SZ, _P]),
    "wq_gemm_grouped_workspace_size": (ctypes.c_int, [ctypes.POINTER(GemmItem), _I32, ctypes.POINTER(_SZ)]),
    "wq_kv_quantize_block": (ctypes.c_int, [_P, _P, ctypes.POINTER(KvCache), _I64, _P]),
    "wq_kv_attention": (ctypes.c_int, [_P, ctypes.POINTER(KvCache), _P, _P, _P, _SZ, _P]),
    "wq_kv_workspace_size": (ctypes.c_int, [ctypes.POINTER(KvCache), ctypes.POINTER(_SZ)]),
    "wq_gemm_nf4": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "wq_gemm_offset": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P]),
    "wq_dequantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P]),
    "wq_gemv_max_batch": (_I32, []),
    "wq_codes_bytes": (ctypes.c_size_t, [_I64, _I64, _I32]),
    "wq_num_groups": (_I64, [_I64, _I64, _I32]),
    "wq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "wq_last_error": (ctypes.c_char_p, []),
    "wq_version": (_I32, []),
}


class WQError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: status {status}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lib = None


def load() -> ctypes.CDLL:
    """Load libwq.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m bit_weight_only_wq_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str):
    if status != WQ_OK:
        lib = load()
        detail = lib.wq_last_error().decode() or lib.wq_status_string(status).decode()
        raise WQError(status, where, detail)
