"""GPU parity of NF4 ("Gör inference billig", the NF4 paragraph): quantize
bit-exact with the oracle (codes and scales; zeros written as +0.0), and the
table-lookup GEMV within the product tolerance of the float64 oracle.  Cases
reach both quantize kernels (team and whole-wave groups), every GEMV tiling
(threads per row x chunks per thread), ragged rows and batch tiles, all-zero
groups, signed zeros, subnormals, +-65504, and weights exactly on a level."""

import numpy as np
import pytest

import oracle.nf4 as onf4
from edge_groups import crafted_groups
from gpu_util import assert_close, bits16, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def check_q(W, group, what):
    device()
    note(f"nf4 quantize {what}: N={W.shape[0]} K={W.shape[1]} G={group}")
    c, s, z = wq.quantize_pack(to_dev(W), group, 4, scheme="nf4")
    oc, os_ = onf4.quantize(W, group)
    assert np.array_equal(bits16(s.cpu().numpy()), bits16(os_)), f"{what}: scales"
    assert np.array_equal(c.cpu().numpy(), oc), f"{what}: codes ({np.sum(c.cpu().numpy() != oc)} bytes)"
    assert not z.cpu().numpy().view(np.uint16).any()
    return (c, s), (oc, os_)


@pytest.mark.parametrize("group", [32, 64, 128, 96, 1024, 1536])
def test_quantize_crafted(group):
    check_q(crafted_groups(group, 4, seed=group + 3), group, "crafted")


@pytest.mark.parametrize("N,K,group", [(1, 32, 32), (65, 512, 64), (7, 4096, 4096), (33, 896, 32),
                                       (300, 8192, 64)])
def test_quantize_random(N, K, group):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 3.0])).astype(np.float16)
    W[0, : min(K, group)] = 0
    check_q(W, group, "random")


def test_quantize_on_levels():
    L = onf4.levels().astype(np.float64)
    rng = np.random.default_rng(8)
    q = rng.integers(0, 16, (16, 128))
    q[:, ::64] = 15
    W = (L[q] * 2.0 ** rng.integers(-10, -2, (16, 1))).astype(np.float16)
    (c, s), _ = check_q(W, 64, "on levels")
    assert np.array_equal(onf4.unpack(c.cpu().numpy(), 128), q)


# K -> chunks C = K/32: <=16 16x1, <=32 16x2, <=64 64x1, <=128 64x2, <=256 64x4, <=512 64x8.
@pytest.mark.parametrize("K,group", [(64, 32), (896, 64), (1536, 64), (4096, 128), (8192, 64),
                                     (11008, 64), (16384, 128)])
@pytest.mark.parametrize("B", [1, 5])
def test_gemm(K, group, B):
    device()
    rng = np.random.default_rng(K + B)
    N = 77
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[3, 7] = 0.6
    X = rng.standard_normal((B, K)).astype(np.float16)
    c, s = onf4.quantize(W, group)
    note(f"nf4 gemm N={N} K={K} G={group} B={B}")
    Y = wq.gemm_nf4(to_dev(X), to_dev(c), to_dev(s), N=N, K=K, group=group)
    assert_close(Y, onf4.gemm(X, c, s, K, group), f"K={K} B={B}")


@pytest.mark.parametrize("B", [2, 9])
def test_gemm_quantized_on_gpu(B):
    device()
    rng = np.random.default_rng(40 + B)
    N, K, G = 1000, 4096, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    (c, s), (oc, os_) = check_q(W, G, "gemm operand")
    Y = wq.gemm_nf4(to_dev(X), c, s, N=N, K=K, group=G)
    assert_close(Y, onf4.gemm(X, oc, os_, K, G), f"B={B}")
