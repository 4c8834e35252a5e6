"""GPU parity of the quad-stream 4x4x4 matrix-core kernel (B = 2..4 on the
automatic path, B = 1..4 on the forced matrix-core path; groups of a multiple
of 64 with an even count per row, matrices of at least 1024 rows;
wq_gemm_qs.hip) against the CPU oracle.

What its geometry makes special, and the shape that exercises it:
  - waves keep one, two or four 512-k positions (K = 4096, 8192, 11008/16384);
    a partial last position reads zero X past K (K = 640, 11008, 256);
  - one to eight row streams per block (K = 256 and 1024 give several);
  - a position's headers are a run from the even group at or below its first
    one (groups of 64, 128, 256, 512: one, two, four or eight positions per
    group, or eight groups per position);
  - a partial last quad (N % 4 != 0) and streams of different lengths;
  - batch rows past B are zero lanes of the A operand (B = 1, 2, 3, 4).
Every output is compared.
"""

import numpy as np
import pytest

import oracle
import wq_inputs
from gpu_util import assert_close, device, note, to_dev, torch

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K, group, batches)
    (1027, 640, 64, (1, 2, 3, 4)),
    (1024, 256, 64, (1, 4)),               # one partial position: eight streams per block
    (2050, 4096, 128, (1, 2, 3, 4)),       # one position per wave
    (3001, 8192, 256, (1, 3, 4)),          # two positions per wave
    (1030, 11008, 128, (1, 2, 4)),         # four per wave, 22 positions, 86 groups per row
    (1024, 16384, 128, (1, 4)),            # four per wave, all 32 positions
    (1025, 2048, 512, (1, 2)),             # two positions per group
    (40000, 1024, 128, (1, 4)),            # four streams per block, long streams
]


@pytest.mark.parametrize("N,K,group,batches", SHAPES)
def test_quad_stream_all_outputs(N, K, group, batches):
    device()
    rng = np.random.default_rng(N + 7 * K + group)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((max(batches), K)).astype(np.float16)
    c, s, z = oracle.quantize(W, group, 4)
    dev = [to_dev(a) for a in (c, s, z)]
    for B in batches:
        ref = oracle.gemm(X[:B], c, s, z, N, K, group, 4)
        note(f"quad-stream N={N} K={K} G={group} B={B}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=group, bits=4, path="mfma", use_workspace=False)
        assert_close(Y, ref, f"N={N} K={K} G={group} B={B}")


def test_quad_stream_repeat_is_bitwise_equal():
    """The waves' sums are added in a fixed order: two calls agree bit for bit."""
    device()
    N, K, G = 4096, 8192, 128
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = to_dev(rng.standard_normal((4, K)).astype(np.float16))
    c, s, z = (to_dev(a) for a in oracle.quantize(W, G, 4))
    for B in (1, 2, 4):
        note(f"quad-stream repeat B={B}")
        a = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=G, bits=4, path="mfma")
        b = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=G, bits=4, path="mfma")
        assert torch.equal(a, b)


def test_quad_stream_on_the_70b_matrix_sampled_rows():
    """The 70B-class up-projection at B = 1, 2, 3, 4: rows sampled across the
    whole matrix (every stream's first and last quads included)."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    c, s, z = wq.quantize_pack(to_dev(W), 128, 4)
    cn, sn, zn = (t.cpu().numpy() for t in (c, s, z))
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(N - 64, N),
                                     np.random.default_rng(5).choice(N, 512, replace=False)]))
    for B in (1, 2, 3, 4):
        note(f"quad-stream {name} B={B}")
        Y = wq.gemm(to_dev(X[:B]), c, s, z, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
        ref = oracle.gemm(X[:B], cn[rows], sn[rows], zn[rows], len(rows), K, 128, 4)
        assert_close(Y[:, rows], ref, f"{name} B={B}")


def test_groups_of_64_past_four_rows_have_no_matrix_core_kernel():
    """Past B = 4 a group of 64 has no matrix-core kernel: the forced path is
    refused, the automatic path takes the GEMV."""
    device()
    N, K = 1024, 640
    W = (np.random.default_rng(4).standard_normal((N, K)) * 0.02).astype(np.float16)
    c, s, z = (to_dev(a) for a in oracle.quantize(W, 64, 4))
    X = to_dev(np.ones((5, K), np.float16))
    with pytest.raises(wq.WQError):
        wq.gemm(X, c, s, z, N=N, K=K, group=64, bits=4, path="mfma")
    Y = wq.gemm(X, c, s, z, N=N, K=K, group=64, bits=4)
    assert Y.shape == (5, N)
