"""GPU parity of the 2- and 3-bit GEMV against the CPU oracle.

Codes are the bit stream of wq_quantize_pack (code k of a row at bits
[k*b, k*b+b)), unpacked in 32-code chunks that each lie in one group.  The
cases reach every (threads per row, units per thread) tiling, ragged rows
(threads past a row's end), ragged row passes and batch tiles (B = 5, 9),
groups of one chunk (32) up to one per row, both scale schemes, and the
70B-class up-projection at full size on sampled rows; the oracle quantizes
and multiplies the same seeded weights on the CPU.
"""

import numpy as np
import pytest

import oracle
import wq_inputs
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_case(N, K, group, bits, B, scheme="asym", seed=0):
    device()
    rng = np.random.default_rng(seed + K + 7 * N + 31 * B + bits)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W.reshape(-1)[rng.choice(N * K, max(1, N * K // 5000), replace=False)] = 0.4
    X = rng.standard_normal((B, K)).astype(np.float16)
    host = oracle.quantize(W, group, bits, scheme=scheme)
    dev = tuple(to_dev(a) for a in host)
    note(f"lowbit gemm b={bits} N={N} K={K} G={group} B={B} {scheme}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=group, bits=bits)
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), f"b={bits} K={K} G={group} B={B}")


# (K, group): units per row U = K/64 (2 bits) or K/128 (3 bits) pick the
# tiling: U <= 16 -> 16x1, <= 32 -> 16x2, <= 64 -> 64x1, <= 128 -> 64x2,
# <= 256 -> 64x4, <= 512 -> 64x8 (2 bits only).
# K = 32768 puts 68-74 KB of X records in LDS (the 128 KB budget; it did not
# fit the old 64 KB).
CASES_2 = [(64, 32), (1024, 32), (1536, 64), (4096, 128), (8192, 128), (8192, 32),
           (12288, 256), (28672, 128), (4096, 4096), (32768, 128)]
CASES_3 = [(128, 32), (896, 32), (4096, 128), (4096, 64), (8192, 128), (11008, 128),
           (28672, 128), (3968, 3968), (32768, 128)]


@pytest.mark.parametrize("K,group", CASES_2)
@pytest.mark.parametrize("B", [1, 5])
def test_two_bit(K, group, B):
    run_case(77, K, group, 2, B)


@pytest.mark.parametrize("K,group", CASES_3)
@pytest.mark.parametrize("B", [1, 5])
def test_three_bit(K, group, B):
    run_case(77, K, group, 3, B)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("B", [2, 9])
@pytest.mark.parametrize("scheme", ["asym", "sym", "sym_tensor"])
def test_schemes_and_batches(bits, B, scheme):
    run_case(1000, 4096, 32 if bits == 2 else 128, bits, B, scheme=scheme)


@pytest.mark.parametrize("bits", [2, 3])
def test_full_size_sampled(bits):
    """The 70B-class up projection (N 28672, K 8192, group 128) at B = 1:
    GPU quantize + GEMM, the oracle on sampled rows."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    cfg = wq_inputs.WORKLOADS[name]
    N, K, G = cfg["N"], cfg["K"], cfg["group"]
    W, X = wq_inputs.workload_arrays(name)
    note(f"lowbit full size b={bits}")
    codes, scales, zeros = wq.quantize_pack(to_dev(W), G, bits)
    Y = wq.gemm(to_dev(X[:1]), codes, scales, zeros, N=N, K=K, group=G, bits=bits)
    rows = np.unique(np.concatenate([np.random.default_rng(40 + bits).choice(N, 384, replace=False),
                                     [0, N - 1]]))
    ref = oracle.gemm(X[:1], *oracle.quantize(W[rows], G, bits), len(rows), K, G, bits)
    assert_close(Y.cpu().numpy()[:, rows].astype(np.float64), ref, f"full size b={bits}")


def test_unsupported_shapes():
    device()
    X = torch.zeros((1, 96), dtype=torch.float16, device="cuda")
    c = torch.zeros((4, 96 * 3 // 8), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 3), dtype=torch.float16, device="cuda")
    with pytest.raises(Exception):
        wq.gemm(X, c, s, s, N=4, K=96, group=32, bits=3)      # K % 128 != 0
    X = torch.zeros((1, 128), dtype=torch.float16, device="cuda")
    c = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(Exception):
        wq.gemm(X, c, s, s, N=4, K=128, group=16, bits=2)      # group % 32 != 0
    with pytest.raises(Exception):
        wq.gemm(X, c, s[:, :4], s[:, :4], N=4, K=128, group=32, bits=2, path="mfma")
