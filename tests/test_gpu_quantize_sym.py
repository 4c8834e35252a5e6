"""GPU parity of the symmetric schemes of wq_quantize_pack_ex against the CPU
oracle (codes, scales and zero points bit-exact), and of wq_gemm on the codes
they produce (to the product tolerance).

Symmetric per group takes the group's absolute maximum (group = K: one scale
per output channel); per tensor takes the whole matrix's, found by two
reduction launches first.  The cases reach every code width 2..8, the team
and whole-wave quantize kernels, both clamp ends, all-zero scopes, a matrix
large enough that the reduction's blocks each cover many chunks (with its
loudest value in the last chunk), and the matrix of "Quantize a matrix by
hand" ("Quantization & inference optimisation")."""

import numpy as np
import pytest

import oracle
from edge_groups import crafted_groups
from gpu_util import assert_close, bits16, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALL_BITS = [2, 3, 4, 5, 6, 7, 8]
SCHEMES = ["sym", "sym_tensor"]


def check_sym(W, group, bits, scheme, what):
    device()
    note(f"quantize {scheme} {what}: N={W.shape[0]} K={W.shape[1]} G={group} b={bits}")
    codes, scales, zeros = wq.quantize_pack(to_dev(W), group, bits, scheme=scheme)
    oc, os_, oz = oracle.quantize(W, group, bits, scheme=scheme)
    gc = codes.cpu().numpy()
    gs = bits16(scales.cpu().numpy())
    gz = bits16(zeros.cpu().numpy())
    assert np.array_equal(gs, bits16(os_)), f"{what}: scales differ ({np.sum(gs != bits16(os_))})"
    assert np.array_equal(gz, bits16(oz)), f"{what}: zeros differ"
    assert np.array_equal(gc, oc), f"{what}: codes differ ({np.sum(gc != oc)} bytes)"
    return (codes, scales, zeros), (oc, os_, oz)


@pytest.mark.parametrize("scheme", SCHEMES)
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("group", [8, 32, 128, 96, 1536])
def test_crafted_groups(scheme, bits, group):
    check_sym(crafted_groups(group, bits, seed=group + 7), group, bits, scheme, "crafted")


@pytest.mark.parametrize("scheme", SCHEMES)
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("N,K,group", [(1, 8, 8), (65, 512, 128), (7, 4096, 4096), (33, 896, 32)])
def test_random_shapes(scheme, bits, N, K, group):
    rng = np.random.default_rng(N * 1000 + K + bits)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 3.0])).astype(np.float16)
    check_sym(W, group, bits, scheme, "random")


@pytest.mark.parametrize("bits", [8, 4, 3])
def test_page_matrix(bits):
    """The 512 x 512 matrix with two loud channels, per channel and per tensor."""
    gen = torch.Generator().manual_seed(0)
    W = torch.randn(512, 512, generator=gen) * 0.02
    W[7] *= 25.0
    W[200] *= 12.0
    W = W.numpy().astype(np.float16)
    check_sym(W, 512, bits, "sym", "page matrix per-channel")
    check_sym(W, 512, bits, "sym_tensor", "page matrix per-tensor")


def test_clamp_ends_and_zero_scopes():
    u = 2.0 ** -24
    W = np.zeros((3, 32), dtype=np.float16)
    W[0, :8] = np.array([-10, 10, 3, -9, 0, -8, 7, 1]) * u
    W[2, 5] = -0.0
    check_sym(W, 8, 4, "sym", "clamp ends / zero groups")
    check_sym(np.zeros((4, 64), dtype=np.float16), 32, 4, "sym_tensor", "all-zero tensor")


@pytest.mark.parametrize("where", ["last", "first"])
def test_tensor_maximum_over_many_blocks(where):
    """4096 x 4104 values: 2.1M chunks over 1024 reduction blocks, the
    loudest value in the first or the last chunk."""
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((4096, 4104)) * 0.02).astype(np.float16)
    if where == "last":
        W[-1, -1] = -3.5
    else:
        W[0, 0] = 2.75
    check_sym(W, 72, 4, "sym_tensor", f"loudest {where}")


@pytest.mark.parametrize("scheme", SCHEMES)
@pytest.mark.parametrize("bits,group", [(4, 128), (8, None)])
@pytest.mark.parametrize("B", [1, 16, 64])
def test_gemm_on_symmetric_codes(scheme, bits, group, B):
    """wq_gemm reads symmetric codes unchanged (zero point 2^(b-1))."""
    rng = np.random.default_rng(B * 10 + bits)
    N, K = 1000, 4096
    G = group or K
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[3] *= 20.0
    X = rng.standard_normal((B, K)).astype(np.float16)
    dev, host = check_sym(W, G, bits, scheme, "gemm operand")
    note(f"gemm on {scheme} codes: B={B} N={N} K={K} G={G} b={bits}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=G, bits=bits)
    assert_close(Y, oracle.gemm(X, *host, N, K, G, bits), f"{scheme} B={B} b={bits}")
