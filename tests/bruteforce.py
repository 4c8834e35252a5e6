"""Exact-rational brute force of the group-wise quantizers.

Written straight from the formulas of "What actually happens when you quantize
a KV cache" (§3 steps 3-5, §4) for the asymmetric codec, and of "Quantization &
inference optimisation" ("Quantize a matrix by hand") for the symmetric one,
with ``fractions.Fraction``; it pins the C oracle on tiny inputs.  It shares nothing with the oracle: fp16 rounding here
is a nearest-neighbour search over the full sorted list of finite fp16 values,
where the oracle constructs the significand arithmetically.

Readings (identical in meaning to the oracle's, arrived at independently):
round half to even; scale rounded once to fp16 and used thereafter; a scale
that rounds to 0 becomes 1.0; zero point stored in fp16, saturating at 65504;
zero point 0 stored as +0.0; codes from the stored zero point; codes packed as
a little-endian bit stream per row.  Symmetric: s = max|x| / (2^(b-1) - 1)
rounded once to fp16 (1.0 if that is 0), signed integers clamped to
[-2^(b-1), 2^(b-1) - 1] and stored offset by 2^(b-1), which is the stored zero
point; one scale per tensor is that scale in every group header.
"""

from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np

# All finite non-negative fp16 values, ascending, with their bit patterns.
_POS_BITS = np.arange(0x0000, 0x7C00, dtype=np.uint16)
_POS_VALS = [Fraction(float(v)) for v in _POS_BITS.view(np.float16)]
FP16_MAX = _POS_VALS[-1]  # 65504


def fp16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def nearest_fp16_bits(v: Fraction) -> int:
    """Bits of the finite fp16 nearest to v >= 0, ties to the even bit pattern.

    Values at or beyond the overflow threshold (65504 + 16) map to 65504.
    """
    assert v >= 0
    if v >= FP16_MAX + 16:
        return 0x7BFF
    i = bisect.bisect_left(_POS_VALS, v)
    if i < len(_POS_VALS) and _POS_VALS[i] == v:
        return int(_POS_BITS[i])
    lo, hi = i - 1, i
    if hi >= len(_POS_VALS):
        return int(_POS_BITS[lo])
    dlo, dhi = v - _POS_VALS[lo], _POS_VALS[hi] - v
    if dlo < dhi:
        return int(_POS_BITS[lo])
    if dhi < dlo:
        return int(_POS_BITS[hi])
    return int(_POS_BITS[lo] if _POS_BITS[lo] % 2 == 0 else _POS_BITS[hi])


def round_half_even(v: Fraction) -> int:
    return round(v)  # Fraction.__round__ rounds half to even


def quantize_group(xbits, bits):
    """xbits: fp16 bit patterns of one group.  Returns (codes, scale_bits, zero_bits)."""
    M = 2 ** bits - 1
    x = [fp16_value(b) for b in xbits]
    mn, mx = min(x), max(x)
    sb = nearest_fp16_bits((mx - mn) / M)
    if sb == 0:
        sb = 0x3C00
    s = fp16_value(sb)
    z = round_half_even(-mn / s)
    if z == 0:
        zb = 0
    else:
        zb = nearest_fp16_bits(Fraction(abs(z)))
        if z < 0:
            zb |= 0x8000
    Z = fp16_value(zb)
    codes = [int(min(max(round_half_even(v / s) + Z, 0), M)) for v in x]
    return codes, sb, zb


def pack_row(codes, bits):
    nbits = len(codes) * bits
    out = bytearray((nbits + 7) // 8)
    for k, q in enumerate(codes):
        for i in range(bits):
            if (q >> i) & 1:
                b = k * bits + i
                out[b // 8] |= 1 << (b % 8)
    return bytes(out)


def quantize(W16: np.ndarray, group: int, bits: int):
    """W16 fp16 [N, K] -> (codes u8, scale bits u16 [N, K/G], zero bits u16)."""
    N, K = W16.shape
    wb = W16.view(np.uint16)
    codes = np.zeros((N, K * bits // 8), dtype=np.uint8)
    sb = np.zeros((N, K // group), dtype=np.uint16)
    zb = np.zeros((N, K // group), dtype=np.uint16)
    for n in range(N):
        row_codes = []
        for g in range(K // group):
            q, s, z = quantize_group([int(v) for v in wb[n, g * group:(g + 1) * group]], bits)
            row_codes += q
            sb[n, g], zb[n, g] = s, z
        codes[n] = np.frombuffer(pack_row(row_codes, bits), dtype=np.uint8)
    return codes, sb, zb


def quantize_group_sym(xbits, bits, amax=None):
    """Symmetric group: (codes, scale_bits, zero_bits).  amax overrides the
    group's own absolute maximum (one scale for the whole tensor)."""
    half = 2 ** (bits - 1)
    x = [fp16_value(b) for b in xbits]
    A = max(abs(v) for v in x) if amax is None else amax
    sb = nearest_fp16_bits(A / (half - 1))
    if sb == 0:
        sb = 0x3C00
    s = fp16_value(sb)
    codes = [int(min(max(round_half_even(v / s), -half), half - 1)) + half for v in x]
    return codes, sb, nearest_fp16_bits(Fraction(half))


def quantize_sym(W16: np.ndarray, group: int, bits: int, per_tensor: bool = False):
    """Symmetric counterpart of quantize(): same outputs and layout."""
    N, K = W16.shape
    wb = W16.view(np.uint16)
    amax = None
    if per_tensor:
        amax = max((abs(fp16_value(int(v))) for v in wb.ravel()), default=Fraction(0))
    codes = np.zeros((N, K * bits // 8), dtype=np.uint8)
    sb = np.zeros((N, K // group), dtype=np.uint16)
    zb = np.zeros((N, K // group), dtype=np.uint16)
    for n in range(N):
        row_codes = []
        for g in range(K // group):
            q, s, z = quantize_group_sym([int(v) for v in wb[n, g * group:(g + 1) * group]],
                                         bits, amax)
            row_codes += q
            sb[n, g], zb[n, g] = s, z
        codes[n] = np.frombuffer(pack_row(row_codes, bits), dtype=np.uint8)
    return codes, sb, zb


def quantize_group_offset(xbits, bits):
    """Float-offset group ("Quantization & inference optimisation",
    "Quantization"): (codes, scale_bits, min_bits) with codes
    round((x - min) / s) clamped to [0, 2^b - 1] and s as for the integer
    zero point."""
    M = 2 ** bits - 1
    x = [fp16_value(b) for b in xbits]
    mn, mx = min(x), max(x)
    sb = nearest_fp16_bits((mx - mn) / M)
    if sb == 0:
        sb = 0x3C00
    s = fp16_value(sb)
    codes = [int(min(round_half_even((v - mn) / s), M)) for v in x]
    mb = nearest_fp16_bits(abs(mn)) | (0x8000 if mn < 0 else 0)
    return codes, sb, mb


def quantize_offset(W16: np.ndarray, group: int, bits: int):
    N, K = W16.shape
    wb = W16.view(np.uint16)
    codes = np.zeros((N, K * bits // 8), dtype=np.uint8)
    sb = np.zeros((N, K // group), dtype=np.uint16)
    mb = np.zeros((N, K // group), dtype=np.uint16)
    for n in range(N):
        row_codes = []
        for g in range(K // group):
            q, s, m = quantize_group_offset([int(v) for v in wb[n, g * group:(g + 1) * group]], bits)
            row_codes += q
            sb[n, g], mb[n, g] = s, m
        codes[n] = np.frombuffer(pack_row(row_codes, bits), dtype=np.uint8)
    return codes, sb, mb
