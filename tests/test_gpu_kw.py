"""GPU parity of the K-split-wave matrix-core kernel (5 <= B <= 64 on
matrices of at least 1.8 16-row tiles per compute unit, group 128,
K = 2048, 4096 or 8192; wq_gemm_kw.hip) against the CPU oracle.

What its geometry makes special, and the shape that exercises it:
  - 2 to 8 tiles per block (N = 7400, 8192, 11008, 12305, 16400, 22000,
    24592, 28672, 40000 on 256 compute units; 40000 needs more blocks than
    compute units);
  - each wave takes a quarter of K (one, two or four two-round steps per wave
    at K = 2048, 4096, 8192), the waves' sums added in LDS;
  - the block's group headers staged in LDS (16, 32 or 64 groups per row);
  - X streamed through a ring of four rounds (B <= 32) or two (B > 32);
  - the last block's tiles past N and a partial last tile (N % 16 != 0);
  - batch rows past B read as zeros from past the end of X (B = 5 .. 64, one,
    two or four 16-row batch blocks);
  - exact-integer code operands with the header applied per round (B <= 16)
    and fp16-dequantized operands (B > 16).
Every output is compared."""

import numpy as np
import pytest

import oracle
import wq_inputs
from gpu_util import assert_close, device, note, to_dev, torch

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K, batches)
    (7400, 4096, (9, 33)),              # 2 tiles per block, last block one partial tile
    (7376, 2048, (5, 16, 64)),          # 461 tiles, the fewest taken: 2 per block, one step per wave
    (8192, 8192, (5, 16, 32, 64)),      # 2 tiles per block, one block per compute unit
    (11990, 2048, (6, 24)),             # 3 tiles per block, partial last tile
    (12305, 2048, (5, 9, 16, 17, 64)),  # 4 tiles per block, partial last tile
    (16400, 4096, (12, 32, 48)),        # 5 tiles per block
    (20000, 4096, (33,)),               # 5 tiles per block
    (22000, 2048, (24,)),               # 6 tiles per block
    (24592, 2048, (64,)),               # 7 tiles per block, partial last block
    (40000, 2048, (8, 9, 64)),          # 8 tiles per block, more blocks than compute units
    (12400, 8192, (16, 24)),            # 4 tiles per block
]


@pytest.mark.parametrize("N,K,batches", SHAPES)
def test_k_split_waves_all_outputs(N, K, batches):
    device()
    rng = np.random.default_rng(N + 13 * K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((max(batches), K)).astype(np.float16)
    c, s, z = oracle.quantize(W, 128, 4)
    dev = [to_dev(a) for a in (c, s, z)]
    for B in batches:
        ref = oracle.gemm(X[:B], c, s, z, N, K, 128, 4)
        note(f"k-split-waves N={N} K={K} B={B}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=128, bits=4, path="mfma", use_workspace=False)
        assert_close(Y, ref, f"N={N} K={K} B={B}")


def test_k_split_waves_repeat_is_bitwise_equal():
    """The waves' sums are added in a fixed order: two calls agree bit for bit."""
    device()
    N, K = 16400, 4096
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = to_dev(rng.standard_normal((64, K)).astype(np.float16))
    c, s, z = (to_dev(a) for a in oracle.quantize(W, 128, 4))
    for B in (10, 32, 64):
        note(f"k-split-waves repeat B={B}")
        a = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=128, bits=4, path="mfma")
        b = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=128, bits=4, path="mfma")
        assert torch.equal(a, b)


@pytest.mark.parametrize("B", [5, 8, 16, 32, 64])
def test_k_split_waves_on_the_70b_matrix_all_rows(B):
    """The 70B-class up-projection (28672 x 8192, the launch the benchmark
    times): every output row against the oracle."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    c, s, z = wq.quantize_pack(to_dev(W), 128, 4)
    cn, sn, zn = (t.cpu().numpy() for t in (c, s, z))
    note(f"k-split-waves {name} B={B}")
    Y = wq.gemm(to_dev(X[:B]), c, s, z, N=N, K=K, group=128, bits=4)
    assert_close(Y, oracle.gemm(X[:B], cn, sn, zn, N, K, 128, 4), f"{name} B={B}")


@pytest.mark.parametrize("B", [8, 16, 24, 64])
def test_k_split_waves_on_the_7b_matrix_all_rows(B):
    """The 7B-class up-projection (11008 x 4096, 0.1 % outliers; three tiles
    per block): every output row against the oracle."""
    device()
    name = "mlp7b_up_k4096_n11008_g128"
    W, _ = wq_inputs.workload_arrays(name)
    N, K = W.shape
    Xb = np.random.default_rng(17).standard_normal((B, K)).astype(np.float16)
    c, s, z = wq.quantize_pack(to_dev(W), 128, 4)
    cn, sn, zn = (t.cpu().numpy() for t in (c, s, z))
    note(f"k-split-waves {name} B={B}")
    Y = wq.gemm(to_dev(Xb), c, s, z, N=N, K=K, group=128, bits=4)
    assert_close(Y, oracle.gemm(Xb, cn, sn, zn, N, K, 128, 4), f"{name} B={B}")
