"""Byte, FLOP and roofline accounting for the group-quantized decode GEMM.

Pure arithmetic, no GPU.  The model is the decode roofline of "Quantization &
inference optimisation" (section "Bandwidth, not compute"): a decode step at
batch B over P weights of w bytes each does 2PB FLOPs and reads Pw bytes, so
its intensity is 2B/w FLOP per byte, independent of P.  The byte count per
weight follows the honest accounting of "What actually happens when you
quantize a KV cache" (§3 step 5 and §5): b/8 bytes of code plus a 4-byte header
(fp16 scale + fp16 zero) per group of G values, i.e. b + 32/G effective bits.
"""

from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_FP16_MFMA_FLOPS = 2.5e15
MI355X_FP32_VALU_FLOPS = 157.3e12
MI355X_COMPUTE_UNITS = 256
MI355X_CLOCK_HZ = 2.4e9

HEADER_BYTES_PER_GROUP = 4  # one fp16 scale + one fp16 zero point


def effective_bits(bits: int, group: int) -> float:
    """Bits per stored value including the per-group header: b + 32/G."""
    return bits + 8.0 * HEADER_BYTES_PER_GROUP / group


def bytes_per_weight(bits: int, group: int) -> float:
    """w in the 2B/w intensity: code bytes plus header bytes per weight."""
    return effective_bits(bits, group) / 8.0


def compression_ratio(bits: int, group: int) -> float:
    """fp16 bytes over quantized bytes (3.76x at b=4, G=128)."""
    return 16.0 / effective_bits(bits, group)


def packed_bytes(N: int, K: int, group: int, bits: int) -> int:
    """Codes plus headers of an [N, K] matrix: N*K*b/8 + 4*N*K/G."""
    return N * K * bits // 8 + HEADER_BYTES_PER_GROUP * N * (K // group)


def gemm_bytes(B: int, N: int, K: int, group: int, bits: int, act_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one Y[B,N] = X[B,K] W_hat[N,K]^T call.

    Packed weights read once, X read once, Y written once (fp16 X and Y).
    """
    return packed_bytes(N, K, group, bits) + act_bytes * B * K + act_bytes * B * N


def quantize_bytes(N: int, K: int, group: int, bits: int) -> int:
    """Algorithmic HBM bytes of quantize/pack: fp16 W read, codes+headers written."""
    return 2 * N * K + packed_bytes(N, K, group, bits)


def gemm_flops(B: int, N: int, K: int) -> int:
    """Useful FLOPs of the product: 2*B*N*K (one multiply-add per weight per row)."""
    return 2 * B * N * K


def intensity(B: int, w_bytes: float) -> float:
    """Decode-step arithmetic intensity 2B/w in FLOP per byte."""
    return 2.0 * B / w_bytes


def ridge_flop_per_byte(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth


def break_even_batch(peak_flops: float, bandwidth: float, w_bytes: float) -> float:
    """Batch at which 2B/w reaches the card's FLOP/byte ratio: ratio * w / 2."""
    return ridge_flop_per_byte(peak_flops, bandwidth) * w_bytes / 2.0


def bytes_read_per_token(params: float, bits: int) -> float:
    """Weight bytes read per decode token for a model of `params` weights."""
    return params * bits / 8.0


def roofline_time_s(bytes_moved: float, flops: float,
                    bandwidth: float = MI355X_HBM_BYTES_PER_S,
                    peak_flops: float = MI355X_FP16_MFMA_FLOPS) -> float:
    """Lower bound on a kernel's time: max(bytes/BW, flops/peak)."""
    return max(bytes_moved / bandwidth, flops / peak_flops)


def kv_cache_bytes(heads: int, tokens: int, head_dim: int = 128, group: int = 128, bits: int = 4) -> int:
    """Quantized KV cache of `heads` heads holding `tokens` tokens each: K and V
    codes plus one 4-byte header per group (K per channel per `group` tokens,
    V per token) -- 136 B per token per head at 4 bits, D = G = 128, the
    "What actually happens when you quantize a KV cache" §5 count."""
    codes = 2 * heads * tokens * head_dim * bits // 8
    k_hdr = HEADER_BYTES_PER_GROUP * heads * head_dim * (tokens // group)
    v_hdr = HEADER_BYTES_PER_GROUP * heads * tokens
    return codes + k_hdr + v_hdr


def kv_attention_bytes(heads: int, tokens: int, head_dim: int = 128) -> int:
    """Algorithmic bytes of one decode-attention step: the whole cache read
    once, the fp16 query read and the fp16 output written."""
    return kv_cache_bytes(heads, tokens, head_dim) + 2 * 2 * heads * head_dim


def kv_append_bytes(heads: int, group: int = 128, head_dim: int = 128) -> int:
    """Quantize-on-append of one block per head: fp16 K and V read, codes and
    headers written."""
    return 2 * 2 * heads * group * head_dim + kv_cache_bytes(heads, group, head_dim, group)
