"""Seeded synthetic inputs for the weight-only group-quantized decode GEMM.

This module only draws random numbers and describes workload shapes. It holds
none of the quantization or matmul arithmetic, so the CPU oracle and the GPU
path can both be fed the same bytes from it without sharing any method code.

Recipe (all draws use ``numpy.random.default_rng``):
  * W ~ N(0, sigma) drawn in float64, scaled by sigma, then cast once to fp16
    (numpy's direct, correctly rounded float64 -> float16 conversion).
  * Optional outliers: ``round(frac * N * K)`` distinct positions chosen with
    ``rng.choice(N*K, k, replace=False)`` are overwritten with +-magnitude, the
    sign drawn by ``rng.integers(0, 2, k)``.  This mirrors the heavy-tailed
    statistics the Swedish inference page measures on a real 896 x 4864 MLP
    matrix (std 0.018, max at 24 sigma), whose shape the first workload copies.
  * X ~ N(0, 1) in float64 cast to fp16, drawn after W from the same generator,
    at the workload's largest batch; smaller batches use its first rows.

The 7B decode-step weight set draws each matrix from its own generator seeded
with ``[seed, layer, matrix_index]`` so any one matrix can be rebuilt alone.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS",
    "DECODE_SET_SHAPES",
    "draw_weights",
    "draw_activations",
    "workload_arrays",
    "decode_set_matrix",
]

# Shapes and distributions of the five workloads. ``batches`` lists the batch
# sizes each one is exercised at.
WORKLOADS = {
    # Single GEMV on the 896 x 4864 MLP matrix shape, group 32 along K.
    "gemv_k896_n4864_g32": dict(
        K=896, N=4864, group=32, bits=4, sigma=0.02, outlier_frac=0.0,
        outlier_mag=0.0, batches=(1,), seed=0),
    # 7B-class MLP up-projection with 0.1% outliers at +-0.5.
    "mlp7b_up_k4096_n11008_g128": dict(
        K=4096, N=11008, group=128, bits=4, sigma=0.02, outlier_frac=0.001,
        outlier_mag=0.5, batches=(1, 4, 8), seed=0),
    # 70B-class MLP up-projection.
    "mlp70b_up_k8192_n28672_g128": dict(
        K=8192, N=28672, group=128, bits=4, sigma=0.015, outlier_frac=0.0,
        outlier_mag=0.0, batches=(1, 16, 64), seed=0),
    # Batch sweep across the ridge point.
    "ridge_sweep_k8192_n8192_g128": dict(
        K=8192, N=8192, group=128, bits=4, sigma=0.02, outlier_frac=0.0,
        outlier_mag=0.0, batches=(1, 2, 4, 8, 16, 32, 64, 128, 256, 512), seed=0),
}

# The 7B decode-step weight set: per layer, (name, N, K) of each projection.
DECODE_SET_SHAPES = (
    ("q", 4096, 4096),
    ("k", 4096, 4096),
    ("v", 4096, 4096),
    ("o", 4096, 4096),
    ("gate", 11008, 4096),
    ("up", 11008, 4096),
    ("down", 4096, 11008),
)
DECODE_SET_LAYERS = 32
DECODE_SET_BATCH = 32
DECODE_SET_SIGMA = 0.02


def draw_weights(rng: np.random.Generator, N: int, K: int, sigma: float,
                 outlier_frac: float = 0.0, outlier_mag: float = 0.0) -> np.ndarray:
    """Return an fp16 [N, K] weight matrix drawn from ``rng`` (see module doc)."""
    w = rng.standard_normal((N, K))
    w *= sigma
    w16 = w.astype(np.float16)
    del w
    if outlier_frac > 0.0:
        k = int(round(outlier_frac * N * K))
        idx = rng.choice(N * K, k, replace=False)
        sign = rng.integers(0, 2, k)
        vals = np.where(sign == 1, outlier_mag, -outlier_mag).astype(np.float16)
        w16.reshape(-1)[idx] = vals
    return w16


def draw_activations(rng: np.random.Generator, B: int, K: int) -> np.ndarray:
    """Return fp16 [B, K] activations ~ N(0, 1)."""
    return rng.standard_normal((B, K)).astype(np.float16)


def workload_arrays(name: str, rows: int | None = None):
    """Draw (W fp16 [N, K], X fp16 [Bmax, K]) for a named workload.

    ``rows`` truncates nothing in the draw order: the full W is drawn and then
    the first ``rows`` rows are returned, so a sample is a prefix of the very
    same matrix.
    """
    cfg = WORKLOADS[name]
    rng = np.random.default_rng(cfg["seed"])
    W = draw_weights(rng, cfg["N"], cfg["K"], cfg["sigma"], cfg["outlier_frac"],
                     cfg["outlier_mag"])
    X = draw_activations(rng, max(cfg["batches"]), cfg["K"])
    if rows is not None:
        W = np.ascontiguousarray(W[:rows])
    return W, X


def decode_set_matrix(layer: int, index: int, seed: int = 0):
    """Draw (W fp16 [N, K], X fp16 [32, K]) for one matrix of the 7B decode set."""
    _, N, K = DECODE_SET_SHAPES[index]
    rng = np.random.default_rng([seed, layer, index])
    W = draw_weights(rng, N, K, DECODE_SET_SIGMA)
    X = draw_activations(rng, DECODE_SET_BATCH, K)
    return W, X
