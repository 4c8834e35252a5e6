"""ctypes view of libwq_probe.so, the HBM read-stream probe (include/wq_probe.h).

A measurement aid: a load-only kernel that gives the read rate the decode
product's roofline fractions are quoted against, beside the vendor peak.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq_probe.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

SIGNATURES = {
    "wq_probe_read": (_I32, [_P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libwq_probe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (python -m bit_weight_only_wq_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def read(buf_ptr: int, rows: int, row_bytes: int, lanes_per_row: int, depth: int, order: int,
         nontemporal: bool, blocks_per_cu: int, sink_ptr: int, stream: int) -> None:
    """Enqueue one read of the [rows, row_bytes] device matrix at buf_ptr."""
    st = load().wq_probe_read(buf_ptr, rows, row_bytes, lanes_per_row, depth, order, int(bool(nontemporal)),
                              blocks_per_cu, sink_ptr, stream)
    if st != 0:
        raise RuntimeError(f"wq_probe_read: status {st}")
