"""GPU parity of wq_dequantize, the reconstruction the products perform in
registers ("Quantization & inference optimisation", section "Quantization":
integer plus the group's endpoints give back an approximate float), written
out as fp32: bit-exact against the oracle's float64 reconstruction rounded to
fp32 for every scheme and width.  The codes come from the oracle's own
quantizers (the GPU quantizer's parity is tested elsewhere), so this checks
the unpacking and the header arithmetic alone.

Why exact: (q - z) * s and level[q] * s are exact in fp32 (at most 17 x 11
and 11 x 11 significant bits), and q * s + m is exact in float64 and one
fused multiply-add in fp32, so both sides round the same exact value once."""

import numpy as np
import pytest

import oracle
from edge_groups import crafted_groups
from gpu_util import device, note, to_dev

import bit_weight_only_wq_amd as wq
from oracle import nf4 as onf4

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = [(1, 8, 8), (33, 256, 32), (65, 512, 128), (7, 4096, 4096), (300, 4096, 128), (17, 896, 64)]


def weights(N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 3.0])).astype(np.float16)
    W[0, :min(K, 8)] = 0.0                      # a group that starts with zeros
    if N > 2:
        W[2, :] = np.float16(1.5)               # a constant row: degenerate groups
    return W


def run(codes, scales, zeros, N, K, group, bits, scheme):
    device()
    note(f"dequantize {scheme} b={bits} N={N} K={K} G={group}")
    out = wq.dequantize(to_dev(codes), to_dev(scales), to_dev(zeros), N, K, group, bits, scheme)
    return out.cpu().numpy()


def check(got, ref, what):
    ref32 = ref.astype(np.float32)
    bad = got.view(np.uint32) != ref32.view(np.uint32)
    assert not bad.any(), f"{what}: {int(bad.sum())} values differ, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("scheme", ["asym", "sym", "sym_tensor"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K,group", SHAPES)
def test_integer_zero_point(scheme, bits, N, K, group):
    W = weights(N, K, seed=N + K + bits)
    c, s, z = oracle.quantize(W, group, bits, scheme=scheme)
    got = run(c, s, z, N, K, group, bits, scheme)
    check(got, oracle.dequantize(c, s, z, N, K, group, bits), f"{scheme} b={bits}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K,group", SHAPES)
def test_float_offset(bits, N, K, group):
    W = weights(N, K, seed=3 * N + K + bits)
    c, s, m = oracle.quantize(W, group, bits, scheme="offset")
    got = run(c, s, m, N, K, group, bits, "offset")
    check(got, oracle.dequantize_offset(c, s, m, K, group, bits), f"offset b={bits}")


@pytest.mark.parametrize("N,K,group", [(1, 32, 32), (33, 256, 32), (65, 512, 64), (7, 4096, 4096),
                                       (300, 4096, 128)])
def test_nf4(N, K, group):
    W = weights(N, K, seed=5 * N + K)
    c, s = onf4.quantize(W, group)
    z = np.zeros_like(s)
    got = run(c, s, z, N, K, group, 4, "nf4")
    check(got, onf4.dequantize(c, s, K, group), "nf4")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_crafted_groups(bits):
    """Groups built to sit on the codec's edges (ties, clamps, subnormal
    scales, constant groups) reconstruct exactly as well."""
    W = crafted_groups(64, bits, seed=bits + 101)
    N, K = W.shape
    c, s, z = oracle.quantize(W, 64, bits)
    check(run(c, s, z, N, K, 64, bits, "asym"), oracle.dequantize(c, s, z, N, K, 64, bits),
          f"crafted b={bits}")
