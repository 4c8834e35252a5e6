"""CPU oracle for decode attention over an int4 KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The product path never imports it.

Source: "What actually happens when you quantize a KV cache" (cited by
section):
  * §1-§2: one decode step scores the new token's query against the key of
    every cached token and takes the softmax-weighted average of their values;
    the running shape is a Llama-2-7B decoder, 32 layers x 32 KV heads of
    dimension 128, fp16.
  * §3 steps 3-5 and §4: the group-wise asymmetric int4 codec (the same codec
    as the weight oracle, ``oracle.quantize``), 4-byte header per group of 128.
  * §7 "axis choice": K is grouped per channel (a group is one channel over
    128 consecutive tokens), V per token (a group is one token's 128-dim
    vector); the newest tokens that do not yet fill a K group stay in fp16.

Cache of one head (the layout the GPU library uses; the oracle produces the
same bytes from the same fp16 inputs):
  per block j of G = 128 tokens:
    kcodes[j]  u8 [G, D/2]   token-major: byte (t, i) holds channels 2i
                             (low nibble) and 2i+1 of token t
    ks[j], kz[j] fp16 [D]    per-channel scale and zero point of the block
    vcodes[j]  u8 [D, G/2]   channel-major: byte (d, i) holds tokens 2i (low
                             nibble) and 2i+1 of channel d
    vs[j], vz[j] fp16 [G]    per-token scale and zero point
  residual: up to G - 1 newest tokens of K and V in fp16, token-major.

Readings (also listed with the other readings of the pages): the V group is
the whole 128-dim token vector; the residual window holds exactly the tokens
past the last full block (K and V alike); attention scale 1/sqrt(D); the
softmax is exact (max-subtracted) in float64.

Parity status: the codec is the pinned weight codec applied along each axis
(checked against the exact-rational brute force on small blocks); attention
is pinned against a library softmax-attention on the dequantized cache and by
closed-form cases (equal scores average V; one dominant score selects its V).
"""

from __future__ import annotations

import numpy as np

from . import quantize as _quantize

BITS = 4


def _unpack_rows(codes: np.ndarray, n: int) -> np.ndarray:
    """u8 rows of two 4-bit codes per byte (even position low) -> int [rows, n]."""
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    out = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out[:, :n]


def _pack_rows(q: np.ndarray) -> np.ndarray:
    """int [rows, n] codes 0..15 -> u8 [rows, n/2], even position in the low nibble."""
    q = q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def quantize_block(Kb: np.ndarray, Vb: np.ndarray):
    """One block of G tokens of one head: Kb, Vb fp16 [G, D] token-major.

    K per channel: each channel's G values are one group (the weight codec on
    Kb^T with group G).  V per token: each token's D values are one group (the
    weight codec on Vb with group D).  Returns the six arrays of the block.
    """
    Kb = np.ascontiguousarray(Kb, dtype=np.float16)
    Vb = np.ascontiguousarray(Vb, dtype=np.float16)
    G, D = Kb.shape
    kc, ks, kz = _quantize(np.ascontiguousarray(Kb.T), G, BITS)      # [D, G/2], [D, 1]
    qk = _unpack_rows(kc, G)                                         # q[d, t]
    vc, vs, vz = _quantize(Vb, D, BITS)                              # [G, D/2], [G, 1]
    qv = _unpack_rows(vc, D)                                         # q[t, d]
    return dict(kcodes=_pack_rows(qk.T), ks=ks[:, 0].copy(), kz=kz[:, 0].copy(),
                vcodes=_pack_rows(qv.T), vs=vs[:, 0].copy(), vz=vz[:, 0].copy())


def dequantize_block(blk) -> tuple[np.ndarray, np.ndarray]:
    """The block's K and V as float64 [G, D]: (q - z) * s with each axis' header."""
    G = blk["vs"].shape[0]
    D = blk["ks"].shape[0]
    qk = _unpack_rows(blk["kcodes"], D)                              # [G, D]
    qv = _unpack_rows(blk["vcodes"], G)                              # [D, G]
    ks = blk["ks"].astype(np.float64)[None, :]
    kz = blk["kz"].astype(np.float64)[None, :]
    vs = blk["vs"].astype(np.float64)[None, :]
    vz = blk["vz"].astype(np.float64)[None, :]
    K = (qk - kz) * ks
    V = ((qv - vz) * vs).T
    return K, V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(K q * scale) V for one head, float64 (§2: score every cached
    key against the query, average the values with the softmax weights)."""
    s = (K.astype(np.float64) @ q.astype(np.float64)) * scale
    if s.size == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    p = np.exp(s - s.max())
    return (p @ V.astype(np.float64)) / p.sum()


def decode_head(q, blocks, k_res, v_res, scale=None) -> np.ndarray:
    """Decode attention of one head over its quantized blocks (in order)
    followed by its fp16 residual tokens."""
    D = q.shape[0]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    Ks, Vs = [], []
    for blk in blocks:
        K, V = dequantize_block(blk)
        Ks.append(K)
        Vs.append(V)
    Ks.append(np.asarray(k_res, dtype=np.float16).astype(np.float64).reshape(-1, D))
    Vs.append(np.asarray(v_res, dtype=np.float16).astype(np.float64).reshape(-1, D))
    return attend(q, np.concatenate(Ks), np.concatenate(Vs), scale)


def cache_bytes_per_token(D: int = 128, G: int = 128, bits: int = BITS) -> float:
    """Quantized bytes of one cached token of one head: K and V codes plus the
    per-token share of the K (per channel, per G tokens) and V (per token)
    headers."""
    return 2 * D * bits / 8 + 4 * D / G + 4
