"""Crafted weight rows that hit the quantizer's corner cases.

Used by the CPU pins (oracle vs exact brute force) and by the GPU parity tests
(HIP path vs oracle).  Each builder returns an fp16 [N, K] matrix whose rows
are made of groups of `group` values.
"""

from __future__ import annotations

import numpy as np

F16 = np.float16


def _f16(vals):
    return np.asarray(vals, dtype=np.float64).astype(F16)


def crafted_groups(group: int, bits: int, seed: int = 1) -> np.ndarray:
    """A stack of single-group rows, one corner case each (K == group)."""
    rng = np.random.default_rng(seed)
    M = 2 ** bits - 1
    G = group
    rows = []

    def add(v):
        v = np.asarray(v, dtype=np.float64)
        if v.size < G:
            v = np.resize(v, G)
        rows.append(v[:G].astype(F16))

    # Exact ties x/s = k + 1/2 with an exactly representable scale: range M*2^-4.
    s = 2.0 ** -4
    tie = [0.0, M * s] + [(k + 0.5) * s for k in range(min(M, G - 2))]
    add(tie)
    # Same with the group shifted negative (ties on the negative side).
    add([-v for v in tie])
    # Negative zero next to positive zero and small values.
    add([-0.0, 0.0, 0.25, -0.125] * (G // 4 + 1))
    # fp16 subnormals only (range of a few subnormal steps: scale may round to 0).
    add(rng.integers(-6, 7, G) * 2.0 ** -24)
    # Subnormals mixed with normals.
    add(np.concatenate([rng.integers(-1023, 1024, G // 2) * 2.0 ** -24,
                        rng.standard_normal(G - G // 2) * 1e-3]))
    # Extreme magnitudes +-65504.
    add([65504.0, -65504.0] + list(rng.standard_normal(G - 2)))
    add([65504.0] * (G // 2) + [-65504.0] * (G - G // 2))
    # Constant groups: zero, positive, negative, subnormal.
    add([0.0] * G)
    add([0.3] * G)
    add([-7.25] * G)
    add([2.0 ** -20] * G)
    # One-signed groups (z negative / beyond M).
    add(np.abs(rng.standard_normal(G)) + 1.0)
    add(-np.abs(rng.standard_normal(G)) - 1.0)
    # Range tiny compared with magnitude: |z| > 2048 (and saturating at b = 8).
    add([1000.0, 1000.5] * (G // 2 + 1))
    add([-1000.0, -999.5] * (G // 2 + 1))
    add([30000.0, 30016.0] * (G // 2 + 1))
    # Two-valued group straddling zero.
    add([-1.0, 1.0] * (G // 2 + 1))
    # Ordinary random groups at the weight distribution of the workloads.
    for _ in range(4):
        add(rng.standard_normal(G) * 0.02)
    # A single outlier in a quiet group (the outlier toy pattern).
    v = rng.standard_normal(G) * 0.02
    v[rng.integers(0, G)] = 4.8
    add(v)
    return np.stack(rows).astype(F16)


def on_grid_matrix(N: int, K: int, group: int, bits: int, seed: int = 2):
    """W built exactly on a quantization grid, with known (s, z, q) per group.

    Scales are powers of two times 3, 5 or 7 and every group uses
    both code 0 and code 2^b-1, so the range is exactly (2^b-1)*s and all
    values (q - z)*s are exact in fp16.  Returns (W fp16, q int, s float, z int).
    """
    rng = np.random.default_rng(seed)
    M = 2 ** bits - 1
    ng = K // group
    s = (rng.integers(1, 4, (N, ng)) * 2 + 1) * 2.0 ** rng.integers(-14, -8, (N, ng))
    z = rng.integers(0, M + 1, (N, ng))
    q = rng.integers(0, M + 1, (N, ng, group))
    q[:, :, 0] = 0
    q[:, :, 1] = M
    W = (q - z[:, :, None]) * s[:, :, None]
    W16 = W.reshape(N, K).astype(F16)
    assert np.array_equal(W16.astype(np.float64), W.reshape(N, K)), "grid not exact in fp16"
    return W16, q.reshape(N, K), s, z
