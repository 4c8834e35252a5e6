"""CPU oracle for the group-quantized decode GEMM (ctypes front end of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The product path never imports this
package and shares no code with it.

What it computes (see oracle.c for the step-by-step citations):
  quantize(W, group, bits)  -> codes u8 [N, K*bits/8], scales fp16, zeros fp16
      group-wise asymmetric quantization along K in exact integer arithmetic,
      following the codec of "What actually happens when you quantize a KV
      cache" §3 steps 3-5 and §4.
  quantize(W, group, bits, scheme="offset") / dequantize_offset / gemm_offset
      the float-offset variant of "Quantization & inference optimisation"
      ("Quantization"): codes round((x - min)/s), x_hat = q*s + min, with the
      group minimum stored in fp16 in place of the zero point.
  quantize(W, group, bits, scheme="sym" | "sym_tensor")
      symmetric absolute-maximum quantization ("Quantization & inference
      optimisation", "Quantize a matrix by hand" and "Per-channel, and what it
      buys"), one scale per group (group = K: per output channel) or one per
      tensor, stored in the same layout with zero point 2^(b-1).
  dequantize(...)           -> W_hat float64 [N, K] = (q - z) * s
  gemm(X, ...)              -> Y_ref float64 [B, N] = X W_hat^T in double.
  kv (submodule)            decode attention over an int4 KV cache: the codec
      above per channel for K and per token for V, dequantized, softmax in
      float64 ("What actually happens when you quantize a KV cache").

Parity status: the quantizer and packer are pinned by the worked groups of
that page and by an exact-rational brute force; the symmetric variant by the
per-tensor/per-channel error table of "Quantize a matrix by hand", the
symmetric step of the KV-cache page's worked group and the same brute force; the GEMM is pinned only by
special cases (on-grid weights against a library matmul, single-row dot
products), since the pages print no GEMM outputs.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_ERRORS = {1: "invalid argument", 2: "non-finite weight", 3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.oracle_quantize.argtypes = [p, i64, i64, i32, i32, p, p, p]
        lib.oracle_quantize_sym.argtypes = [p, i64, i64, i32, i32, i32, p, p, p]
        lib.oracle_quantize_offset.argtypes = [p, i64, i64, i32, i32, p, p, p]
        lib.oracle_dequantize.argtypes = [p, p, p, i64, i64, i32, i32, p]
        lib.oracle_gemm.argtypes = [p, p, p, p, i64, i64, i64, i32, i32, p]
        lib.oracle_gemm_rows.argtypes = [p, p, p, p, i64, i64, i64, i32, i32, p, i64, p]
        for f in (lib.oracle_quantize, lib.oracle_quantize_sym, lib.oracle_quantize_offset,
                  lib.oracle_dequantize,
                  lib.oracle_gemm,
                  lib.oracle_gemm_rows):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (for timing; results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


SCHEMES = ("asym", "sym", "sym_tensor", "offset")


def quantize(W: np.ndarray, group: int, bits: int, scheme: str = "asym"):
    """W fp16 [N, K] -> (codes u8 [N, K*bits//8], scales fp16 [N, K//group], zeros fp16).

    scheme "asym": min/max per group; "sym": absolute maximum per group;
    "sym_tensor": one absolute maximum over the whole matrix; "offset": the
    float-offset variant, whose third array holds the group minima (fp16)
    instead of zero points (dequantize with dequantize_offset).
    """
    if scheme not in SCHEMES:
        raise ValueError(f"oracle: unknown scheme {scheme!r}")
    W = np.ascontiguousarray(W, dtype=np.float16)
    N, K = W.shape
    if K % group or (K * bits) % 8:
        raise ValueError("oracle: invalid argument")
    codes = np.zeros((N, K * bits // 8), dtype=np.uint8)
    scales = np.zeros((N, K // group), dtype=np.float16)
    zeros = np.zeros((N, K // group), dtype=np.float16)
    lib = _load()
    if scheme == "asym":
        rc = lib.oracle_quantize(_ptr(W), N, K, group, bits, _ptr(codes), _ptr(scales),
                                 _ptr(zeros))
    elif scheme == "offset":
        rc = lib.oracle_quantize_offset(_ptr(W), N, K, group, bits, _ptr(codes), _ptr(scales),
                                        _ptr(zeros))
    else:
        rc = lib.oracle_quantize_sym(_ptr(W), N, K, group, bits, int(scheme == "sym_tensor"),
                                     _ptr(codes), _ptr(scales), _ptr(zeros))
    _check(rc)
    return codes, scales, zeros


def dequantize(codes, scales, zeros, N: int, K: int, group: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float16)
    zeros = np.ascontiguousarray(zeros, dtype=np.float16)
    out = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_dequantize(_ptr(codes), _ptr(scales), _ptr(zeros), N, K,
                                     group, bits, _ptr(out)))
    return out


def gemm(X, codes, scales, zeros, N: int, K: int, group: int, bits: int,
         rows=None) -> np.ndarray:
    """Y_ref float64 [B, N] (or [B, len(rows)] for a row sample)."""
    X = np.ascontiguousarray(X, dtype=np.float16)
    B = X.shape[0]
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float16)
    zeros = np.ascontiguousarray(zeros, dtype=np.float16)
    if codes.size != N * K * bits // 8 or scales.size != N * (K // group) \
            or zeros.size != N * (K // group) or X.shape[1] != K:
        raise ValueError("oracle: shape mismatch")
    lib = _load()
    if rows is None:
        Y = np.empty((B, N), dtype=np.float64)
        _check(lib.oracle_gemm(_ptr(X), _ptr(codes), _ptr(scales), _ptr(zeros), B, K, N,
                               group, bits, _ptr(Y)))
        return Y
    r = np.ascontiguousarray(rows, dtype=np.int64)
    Y = np.empty((B, r.size), dtype=np.float64)
    _check(lib.oracle_gemm_rows(_ptr(X), _ptr(codes), _ptr(scales), _ptr(zeros), B, K, N,
                                group, bits, _ptr(r), r.size, _ptr(Y)))
    return Y


def _unpack_codes(codes: np.ndarray, K: int, bits: int) -> np.ndarray:
    bitsarr = np.unpackbits(np.ascontiguousarray(codes, dtype=np.uint8), axis=1,
                            bitorder="little")[:, :K * bits]
    w = 1 << np.arange(bits, dtype=np.int64)
    return (bitsarr.reshape(codes.shape[0], K, bits).astype(np.int64) * w).sum(-1)


def dequantize_offset(codes, scales, mins, K: int, group: int, bits: int) -> np.ndarray:
    """Float-offset variant: W_hat float64 [N, K] = q * s + min (exact in
    double: q * s has at most 19 significant bits)."""
    q = _unpack_codes(codes, K, bits)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=1)
    m = np.repeat(np.asarray(mins, dtype=np.float16).astype(np.float64), group, axis=1)
    return q * s + m


def gemm_offset(X, codes, scales, mins, K: int, group: int, bits: int) -> np.ndarray:
    """Y_ref float64 [B, N] = X W_hat^T for the float-offset variant."""
    return np.asarray(X, dtype=np.float16).astype(np.float64) @ \
        dequantize_offset(codes, scales, mins, K, group, bits).T
