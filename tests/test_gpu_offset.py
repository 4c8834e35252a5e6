"""GPU parity of the float-offset variant ("Quantization & inference
optimisation", section "Quantization": codes round((x - min)/s), x_hat =
q*s + min): quantize bit-exact with the oracle for every width 2..8 (both
quantize kernels), and wq_gemm_offset within the product tolerance for
bits 2, 3, 4 and 8 across the GEMV tilings, ragged rows and batch tiles."""

import numpy as np
import pytest

import oracle
from edge_groups import crafted_groups
from gpu_util import assert_close, bits16, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALL_BITS = [2, 3, 4, 5, 6, 7, 8]


def check_q(W, group, bits, what):
    device()
    note(f"offset quantize {what}: N={W.shape[0]} K={W.shape[1]} G={group} b={bits}")
    c, s, m = wq.quantize_pack(to_dev(W), group, bits, scheme="offset")
    oc, os_, om = oracle.quantize(W, group, bits, scheme="offset")
    assert np.array_equal(bits16(s.cpu().numpy()), bits16(os_)), f"{what}: scales"
    assert np.array_equal(bits16(m.cpu().numpy()), bits16(om)), f"{what}: minima"
    assert np.array_equal(c.cpu().numpy(), oc), f"{what}: codes ({np.sum(c.cpu().numpy() != oc)} bytes)"
    return (c, s, m), (oc, os_, om)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("group", [8, 32, 128, 96, 1536])
def test_quantize_crafted(bits, group):
    check_q(crafted_groups(group, bits, seed=group + 11), group, bits, "crafted")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("N,K,group", [(1, 8, 8), (65, 512, 128), (7, 4096, 4096), (33, 896, 32)])
def test_quantize_random(bits, N, K, group):
    rng = np.random.default_rng(N * 7 + K + bits)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 3.0])).astype(np.float16)
    check_q(W, group, bits, "random")


CASES = {2: [(64, 32), (1536, 64), (8192, 128), (16384, 128)],
         3: [(128, 32), (896, 32), (4096, 128), (11008, 128)],
         4: [(32, 32), (512, 32), (1536, 64), (4096, 128), (8192, 128), (16384, 128)],
         8: [(32, 32), (1024, 32), (4096, 128), (8192, 4096)]}


@pytest.mark.parametrize("bits,K,group", [(b, K, g) for b, v in CASES.items() for K, g in v])
@pytest.mark.parametrize("B", [1, 5])
def test_gemm_offset(bits, K, group, B):
    device()
    rng = np.random.default_rng(bits * 1000 + K + B)
    N = 77
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[5, 3] = 0.7
    X = rng.standard_normal((B, K)).astype(np.float16)
    host = oracle.quantize(W, group, bits, scheme="offset")
    note(f"gemm_offset b={bits} N={N} K={K} G={group} B={B}")
    Y = wq.gemm_offset(to_dev(X), *(to_dev(a) for a in host), N=N, K=K, group=group, bits=bits)
    assert_close(Y, oracle.gemm_offset(X, *host, K, group, bits), f"b={bits} K={K} B={B}")


def test_gemm_offset_quantized_on_gpu():
    device()
    rng = np.random.default_rng(77)
    N, K, G = 1000, 4096, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((9, K)).astype(np.float16)
    dev, host = check_q(W, G, 4, "gemm operand")
    Y = wq.gemm_offset(to_dev(X), *dev, N=N, K=K, group=G, bits=4)
    assert_close(Y, oracle.gemm_offset(X, *host, K, G, 4), "gpu-quantized")
