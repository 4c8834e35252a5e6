"""CPU oracle for NF4 weights: sixteen normal-quantile levels with one
absolute-maximum scale per group, and the dequantize-then-multiply product.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The product path never imports it.

Source: "Gör inference billig: KV cache, batching och kvantisering" (the
paragraph on NF4 after the group-wise absolute-maximum scales): the sixteen
levels are the quantiles of a normal distribution, dense near zero; the
block scaling is the same absolute-maximum scaling as the symmetric scheme,
at blocks of 64 (4.25 bits per weight).

Readings (the page gives no formula):
  * level i (0..15) is the standard normal quantile at probability
    (i + 1/2) / 16, divided by the largest magnitude so that the levels span
    [-1, 1]; the levels are stored in fp16, and every later step uses the
    fp16 values (the set is symmetric and has no exact zero);
  * the scale of a group is its largest |w|, stored in fp16 (exact: it is one
    of the fp16 inputs), 1.0 for an all-zero group;
  * a weight's code is the level nearest to the exact quotient w / s (an
    exact-rational decision, like every decision of the integer codec); a
    quotient exactly between two levels takes the lower code.  Midpoints of
    adjacent fp16 levels have at most 12 significant bits, so a midpoint
    times an fp16 scale is exact in fp32 and w can be compared with it
    directly;
  * codes are packed two per byte, even k in the low nibble (the layout of
    the 4-bit integer codes); dequantization is level[q] * s.

Parity status: the level set is pinned by an empirical-quantile check on a
large normal sample and by symmetry; the encoder by an exact-rational brute
force and by an on-level fixpoint; the product by the dequantize definition
against a library matmul.  The page's NF4 error (0.0952) is measured on real
weights, so it is not reproduced (parity unpinned for that figure).
"""

from __future__ import annotations

import numpy as np


def levels_f64() -> np.ndarray:
    from scipy.stats import norm
    q = norm.ppf((np.arange(16) + 0.5) / 16.0)
    return q / np.abs(q).max()


def levels() -> np.ndarray:
    """The sixteen levels as fp16 (what both the encoder and decoder use)."""
    return levels_f64().astype(np.float16)


def midpoints() -> np.ndarray:
    """fp32 midpoints of adjacent fp16 levels (exact)."""
    L = levels().astype(np.float64)
    mid = (L[:-1] + L[1:]) / 2.0
    m32 = mid.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mid)
    return m32


def quantize(W: np.ndarray, group: int):
    """W fp16 [N, K] -> (codes u8 [N, K/2], scales fp16 [N, K/group])."""
    W = np.ascontiguousarray(W, dtype=np.float16)
    N, K = W.shape
    if K % group or group % 2:
        raise ValueError("nf4: K must be a multiple of group, group even")
    g = W.reshape(N, K // group, group).astype(np.float64)
    s = np.abs(g).max(axis=2)
    s = np.where(s == 0, 1.0, s).astype(np.float16)
    # Thresholds mid_i * s are exact in float64 (and in fp32); the code is the
    # number of thresholds strictly below w.
    th = midpoints().astype(np.float64)[None, None, :] * s.astype(np.float64)[:, :, None]
    q = (g[:, :, :, None] > th[:, :, None, :]).sum(axis=3).reshape(N, K).astype(np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s


def unpack(codes: np.ndarray, K: int) -> np.ndarray:
    q = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.int64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return q[:, :K]


def dequantize(codes: np.ndarray, scales: np.ndarray, K: int, group: int) -> np.ndarray:
    """W_hat float64 [N, K] = level[q] * s."""
    q = unpack(np.asarray(codes, dtype=np.uint8), K)
    L = levels().astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=1)
    return L[q] * s


def gemm(X: np.ndarray, codes: np.ndarray, scales: np.ndarray, K: int, group: int) -> np.ndarray:
    """Y_ref float64 [B, N] = X W_hat^T."""
    return np.asarray(X, dtype=np.float16).astype(np.float64) @ dequantize(codes, scales, K, group).T
