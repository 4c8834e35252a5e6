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

__all__ = ["quantize_pack", "gemm", "gemm_grouped", "gemm_workspace_bytes", "codes_bytes", "num_groups",
           "gemv_max_batch",
           "gemm_nf4", "gemm_offset", "KVCache", "kv_quantize_block", "kv_attention", "WQError", "LIB_PATH", "load"]

_PATHS = {"auto": WQ_PATH_AUTO, "gemv": WQ_PATH_GEMV, "mfma": WQ_PATH_MFMA}


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _size_t(query, *args, where=""):
    """Bytes from a wq_*_workspace_size query (raises on its error status)."""
    import ctypes
    n = ctypes.c_size_t(0)
    check(query(*args, ctypes.byref(n)), where)
    return int(n.value)


def _workspace(nbytes, device, workspace=None):
    """(pointer, bytes, tensor) of a caller workspace: the given uint8 tensor
    (checked against nbytes) or a fresh one from torch's allocator, (None, 0,
    None) when the call needs none.  A fresh tensor goes back to torch's stream-ordered cache
    when the caller drops it, so reuse by later work on the stream is safe."""
    import torch
    if nbytes == 0:
        return None, 0, None
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.device != torch.device(device)
          or workspace.dtype != torch.uint8 or not workspace.is_contiguous()
          or workspace.numel() < nbytes):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {nbytes} bytes on {device}")
    return workspace.data_ptr(), workspace.numel(), workspace


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


def gemm_workspace_bytes(B: int, K: int, N: int, group: int = 128, bits: int = 4, path: str = "auto") -> int:
    """Workspace bytes of a gemm() call of this shape on the current device."""
    return _size_t(load().wq_gemm_workspace_size, B, K, N, group, bits, _PATHS[path], where="wq_gemm")


SCHEMES = {"asym": 0, "sym": 1, "sym_tensor": 2, "nf4": 3, "offset": 4}


def quantize_pack(W, group: int = 128, bits: int = 4, out=None, scheme: str = "asym"):
    """W fp16 [N, K] (GPU) -> (codes u8 [N, K*bits//8], scales fp16 [N, K//group], zeros fp16).

    scheme "asym" (min/max, integer zero point), "sym" (absolute maximum per
    group; group = K for one scale per output channel), "sym_tensor" (one
    absolute maximum for the whole matrix), "nf4" (normal-quantile levels,
    bits = 4; multiply with gemm_nf4) or "offset" (the group minimum as a
    float offset in the third array; multiply with gemm_offset)."""
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
        need = _size_t(lib.wq_quantize_workspace_size, N, K, group, bits, SCHEMES[scheme],
                       where="wq_quantize_pack")
        ws, ws_bytes, _keep = _workspace(need, W.device)
        st = lib.wq_quantize_pack_ex(W.data_ptr(), N, K, group, bits, SCHEMES[scheme],
                                     codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                     ws, ws_bytes, _stream_handle(W.device))
    check(st, "wq_quantize_pack")
    return codes, scales, zeros


def gemm_grouped(items, workspace=None, use_workspace=True):
    """Several products in one call: items is a sequence of
    (X, codes, scales, zeros, N, K, group, bits[, out]) tuples; returns the Y
    tensors in order (each what gemm() gives for its item, within the product
    tolerance).  The call's workspace comes from torch (or `workspace`, a
    uint8 tensor); use_workspace=False runs the plans that need none."""
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
        need = _size_t(lib.wq_gemm_grouped_workspace_size, arr, len(items),
                       where="wq_gemm_grouped") if use_workspace else 0
        ws, ws_bytes, _keep = _workspace(need, dev, workspace)
        st = lib.wq_gemm_grouped(arr, len(items), ws, ws_bytes, _stream_handle(dev))
    check(st, "wq_gemm_grouped")
    return outs


def gemm(X, codes, scales, zeros, N: int, K: int, group: int = 128, bits: int = 4,
         path: str = "auto", out=None, workspace=None, use_workspace=True):
    """Y fp16 [B, N] = X fp16 [B, K] times the dequantized [N, K] matrix, transposed.

    The call's workspace (wq_gemm_workspace_size bytes) comes from torch, or
    from `workspace` (a uint8 tensor); use_workspace=False runs the plan that
    needs none (wq_gemm's)."""
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
        need = _size_t(lib.wq_gemm_workspace_size, B, K, N, group, bits, _PATHS[path],
                       where="wq_gemm") if use_workspace else 0
        ws, ws_bytes, _keep = _workspace(need, X.device, workspace)
        st = lib.wq_gemm_ex(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                            out.data_ptr(), B, K, N, group, bits, _PATHS[path], ws, ws_bytes,
                            _stream_handle(X.device))
    check(st, "wq_gemm")
    return out


class KVCache:
    """Caller-owned buffers of an int4 KV cache (head dimension 128, blocks of
    128 tokens), as torch tensors on one GPU; layout as wq_kv_cache in wq.h."""

    D = 128
    G = 128

    def __init__(self, heads: int, max_blocks: int, device="cuda"):
        import torch
        u8, f16 = torch.uint8, torch.float16
        H, NB, D, G = heads, max_blocks, self.D, self.G
        self.heads, self.max_blocks = heads, max_blocks
        self.kcodes = torch.zeros((H, NB, G, D // 2), dtype=u8, device=device)
        self.kscales = torch.zeros((H, NB, D), dtype=f16, device=device)
        self.kzeros = torch.zeros((H, NB, D), dtype=f16, device=device)
        self.vcodes = torch.zeros((H, NB, D, G // 2), dtype=u8, device=device)
        self.vscales = torch.zeros((H, NB * G), dtype=f16, device=device)
        self.vzeros = torch.zeros((H, NB * G), dtype=f16, device=device)
        self.kres = torch.zeros((H, G, D), dtype=f16, device=device)
        self.vres = torch.zeros((H, G, D), dtype=f16, device=device)

    @property
    def device(self):
        return self.kcodes.device

    def descriptor(self):
        from ._lib import KvCache
        return KvCache(self.kcodes.data_ptr(), self.kscales.data_ptr(), self.kzeros.data_ptr(),
                       self.vcodes.data_ptr(), self.vscales.data_ptr(), self.vzeros.data_ptr(),
                       self.kres.data_ptr(), self.vres.data_ptr(), self.heads, self.max_blocks)


def kv_quantize_block(K, V, cache: KVCache, block: int):
    """K, V fp16 [heads, 128, 128] (token-major) -> block `block` of every head."""
    import ctypes
    import torch
    shape = (cache.heads, cache.G, cache.D)
    _need(K, torch.float16, shape, "K")
    _need(V, torch.float16, shape, "V")
    desc = cache.descriptor()
    with torch.cuda.device(cache.device):
        st = load().wq_kv_quantize_block(K.data_ptr(), V.data_ptr(), ctypes.byref(desc), block,
                                         _stream_handle(cache.device))
    check(st, "wq_kv_quantize_block")


def kv_attention(q, cache: KVCache, lens, out=None, workspace=None, use_workspace=True):
    """q fp16 [heads, 128], lens int32 [heads] (GPU) -> out fp16 [heads, 128].
    The call's workspace (context-split partials) comes from torch or from
    `workspace`; use_workspace=False runs one workgroup per head."""
    import ctypes
    import torch
    _need(q, torch.float16, (cache.heads, cache.D), "q")
    _need(lens, torch.int32, (cache.heads,), "lens")
    if out is None:
        out = torch.empty((cache.heads, cache.D), dtype=torch.float16, device=q.device)
    _need(out, torch.float16, (cache.heads, cache.D), "out")
    desc = cache.descriptor()
    lib = load()
    with torch.cuda.device(cache.device):
        need = _size_t(lib.wq_kv_workspace_size, ctypes.byref(desc), where="wq_kv_attention") \
            if use_workspace else 0
        ws, ws_bytes, _keep = _workspace(need, cache.device, workspace)
        st = lib.wq_kv_attention(q.data_ptr(), ctypes.byref(desc), lens.data_ptr(), out.data_ptr(),
                                 ws, ws_bytes, _stream_handle(cache.device))
    check(st, "wq_kv_attention")
    return out


def gemm_nf4(X, codes, scales, N: int, K: int, group: int = 64, out=None):
    """Y fp16 [B, N] = X [B, K] times the NF4 weights (codes, scales from
    quantize_pack(..., scheme="nf4"))."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be 2-D [B, K]")
    B = X.shape[0]
    _need(X, torch.float16, (B, K), "X")
    _need(codes, torch.uint8, (N, K // 2), "codes")
    _need(scales, torch.float16, (N, K // group), "scales")
    if out is None:
        out = torch.empty((B, N), dtype=torch.float16, device=X.device)
    _need(out, torch.float16, (B, N), "out")
    with torch.cuda.device(X.device):
        st = load().wq_gemm_nf4(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), out.data_ptr(),
                                B, K, N, group, _stream_handle(X.device))
    check(st, "wq_gemm_nf4")
    return out


def gemm_offset(X, codes, scales, mins, N: int, K: int, group: int = 128, bits: int = 4, out=None):
    """Y fp16 [B, N] for float-offset weights (quantize_pack(..., scheme="offset"))."""
    import torch
    if X.dim() != 2:
        raise ValueError("X must be 2-D [B, K]")
    B = X.shape[0]
    _need(X, torch.float16, (B, K), "X")
    _need(codes, torch.uint8, (N, K * bits // 8), "codes")
    _need(scales, torch.float16, (N, K // group), "scales")
    _need(mins, torch.float16, (N, K // group), "mins")
    if out is None:
        out = torch.empty((B, N), dtype=torch.float16, device=X.device)
    _need(out, torch.float16, (B, N), "out")
    with torch.cuda.device(X.device):
        st = load().wq_gemm_offset(X.data_ptr(), codes.data_ptr(), scales.data_ptr(), mins.data_ptr(),
                                   out.data_ptr(), B, K, N, group, bits, _stream_handle(X.device))
    check(st, "wq_gemm_offset")
    return out


def dequantize(codes, scales, zeros, N: int, K: int, group: int = 128, bits: int = 4,
               scheme: str = "asym", out=None):
    """fp32 [N, K] weights reconstructed from quantize_pack(..., scheme) output
    (a test aid: the products reconstruct in registers)."""
    import torch
    if scheme not in SCHEMES:
        raise ValueError(f"unknown scheme {scheme!r}")
    _need(codes, torch.uint8, (N, K * bits // 8), "codes")
    _need(scales, torch.float16, (N, K // group), "scales")
    _need(zeros, torch.float16, (N, K // group), "zeros")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, (N, K), "out")
    with torch.cuda.device(codes.device):
        st = load().wq_dequantize(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, group,
                                  bits, SCHEMES[scheme], out.data_ptr(), _stream_handle(codes.device))
    check(st, "wq_dequantize")
    return out
