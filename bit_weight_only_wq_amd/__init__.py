"""MI355X-native weight-only group-quantized decode GEMM.

Python binding of libwq.so (C ABI in include/wq.h).  This layer only turns
torch tensors and the current HIP stream into raw pointers; every step of the
computation runs in the HIP kernels, and there is no CPU fallback: if the
library is not built, the calls raise.

    codes, scales, zeros = quantize_pack(W, group=128, bits=4)   # W fp16 [N, K] on the GPU
    Y = gemm(X, codes, scales, zeros, N=N, K=K, group=128, bits=4)  # X fp16 [B, K]
"""

from __future__ import annotations

from . import roofline  # noqa: F401  (pure arithmetic, no GPU)
from ._lib import (WQ_PATH_AUTO, WQ_PATH_GEMV, WQ_PATH_MFMA, WQError,  # noqa: F401
                   LIB_PATH, check, load)

__all__ = ["quantize_pack", "gemm", "codes_bytes", "num_groups", "gemv_max_batch",
           "WQError", "LIB_PATH", "load"]

_PATHS = {"auto": WQ_PATH_AUTO, "gemv": WQ_PATH_GEMV, "mfma": WQ_PATH_MFMA}


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, dtype, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def codes_bytes(N: int, K: int, bits: int) -> int:
    return int(load().wq_codes_bytes(N, K, bits))


def num_groups(N: int, K: int, group: int) -> int:
    return int(load().wq_num_groups(N, K, group))


def gemv_max_batch() -> int:
    return int(load().wq_gemv_max_batch())


SCHEMES = {"asym": 0, "sym": 1, "sym_tensor": 2}


def quantize_pack(W, group: int = 128, bits: int = 4, out=None, scheme: str = "asym"):
    """W fp16 [N, K] (GPU) -> (codes u8 [N, K*bits//8], scales fp16 [N, K//group], zeros fp16).

    scheme "asym" (min/max, integer zero point), "sym" (absolute maximum per
    group; group = K for one scale per output channel) or "sym_tensor" (one
    absolute maximum for the whole matrix)."""
    import torch
    lib = load()
    if scheme not in SCHEMES:
        raise ValueError(f"unknown scheme {scheme!r}")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    N, K = W.shape
    _need(W, torch.float16, (N, K), "W")
    if K % group or (K * bits) % 8:
        raise ValueError("K must be a multiple of group and of 8/bits")
    if out is None:
        codes = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=W.device)
        scales = torch.empty((N, K // group), dtype=torch.float16, device=W.device)
        zeros = torch.empty((N, K // group), dtype=torch.float16, device=W.device)
    else:
        codes, scales, zeros = out
        _need(codes, torch.uint8, (N, K * bits // 8), "codes")
        _need(scales, torch.float16, (N, K // group), "scales")
        _need(zeros, torch.float16, (N, K // group), "zeros")
    with torch.cuda.device(W.device):
        st = lib.wq_quantize_pack_ex(W.data_ptr(), N, K, group, bits, SCHEMES[scheme],
                                     codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                     _stream_handle(W.device))
    check(st, "wq_quantize_pack")
    return codes, scales, zeros


def gemm_grouped(items):
    """Several products in one call: items is a sequence of
    (X, codes, scales, zeros, N, K, group, bits[, out]) tuples; returns the Y
    tensors in order (each exactly what gemm() gives for its item)."""
    import ctypes
    import torch
    from ._lib import GemmItem
    lib = load()
    arr = (GemmItem * max(len(items), 1))()
    outs = []
    dev = None
    for i, it in enumerate(items):
        X, codes, scales, zeros, N, K, group, bits = it[:8]
        out = it[8] if len(it) > 8 else None
        if X.dim() != 2:
            raise ValueError("X must be 2-D [B, K]")
        B = X.shape[0]
        _need(X, torch.float16, (B, K), "X")
        _need(codes, torch.uint8, (N, K * bits // 8), "codes")
        _need(scales, torch.float16, (N, K // group), "scales")
        _need(zeros, torch.float16, (N, K // group), "zeros")
        if dev is None:
            dev = X.device
        elif X.device != dev:
            raise ValueError("all items must be on one device")
        if out is None:
            out = torch.empty((B, N), dtype=torch.float16, device=X.device)
        else:
            _need(out, torch.float16, (B, N), "out")
        outs.append(out)
        arr[i] = GemmItem(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                          out.data_ptr(), B, K, N, group, bits)
    if not items:
        return outs
    with torch.cuda.device(dev):
        st = lib.wq_gemm_grouped(arr, len(items), _stream_handle(dev))
    check(st, "wq_gemm_grouped")
    return outs


def gemm(X, codes, scales, zeros, N: int, K: int, group: int = 128, bits: int = 4,
         path: str = "auto", out=None):
    """Y fp16 [B, N] = X fp16 [B, K] times the dequantized [N, K] matrix, transposed."""
    import torch
    lib = load()
    if X.dim() != 2:
        raise ValueError("X must be 2-D [B, K]")
    B = X.shape[0]
    _need(X, torch.float16, (B, K), "X")
    _need(codes, torch.uint8, (N, K * bits // 8), "codes")
    _need(scales, torch.float16, (N, K // group), "scales")
    _need(zeros, torch.float16, (N, K // group), "zeros")
    if out is None:
        out = torch.empty((B, N), dtype=torch.float16, device=X.device)
    else:
        _need(out, torch.float16, (B, N), "out")
    with torch.cuda.device(X.device):
        st = lib.wq_gemm_ex(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                            out.data_ptr(), B, K, N, group, bits, _PATHS[path],
                            _stream_handle(X.device))
    check(st, "wq_gemm")
    return out
