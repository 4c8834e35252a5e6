"""GPU parity of the tile-stream 16x16x32 matrix-core kernel (B <= 16 on
matrices of at least 2048 rows, group 128, K % 512 == 0, K <= 8192;
wq_gemm_ts.hip) against the CPU oracle.

What its geometry makes special, and the shape that exercises it:
  - waves keep one or two 512-k positions (K = 4096; K = 6144, 8192) and
    walk their tiles position by position, the second pass adding to the
    first's sums;
  - several row streams per block (K = 512, 1024, 2048);
  - a partial last tile (N % 16 != 0) and streams of different lengths;
  - batch rows past B are zero rows of the A operand (B = 5 .. 16);
  - header arrays not 8-byte aligned go to another kernel.
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
    (2085, 4096, 128, (5, 8, 13, 16)),     # one position per wave, partial last tile
    (4100, 8192, 128, (5, 9, 16)),         # two positions per wave
    (2061, 6144, 128, (6, 16)),            # 12 positions: four waves with two, four with one
    (2560, 512, 128, (8, 16)),             # one position: eight streams per block
    (3000, 2048, 128, (7, 16)),            # two streams per block
    (33 * 256 * 16 + 5, 1024, 128, (12,)),  # long streams, four streams per block
]


@pytest.mark.parametrize("N,K,group,batches", SHAPES)
def test_tile_stream_all_outputs(N, K, group, batches):
    device()
    rng = np.random.default_rng(N + 11 * K + group)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((max(batches), K)).astype(np.float16)
    c, s, z = oracle.quantize(W, group, 4)
    dev = [to_dev(a) for a in (c, s, z)]
    for B in batches:
        ref = oracle.gemm(X[:B], c, s, z, N, K, group, 4)
        note(f"tile-stream N={N} K={K} G={group} B={B}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=group, bits=4, path="mfma", use_workspace=False)
        assert_close(Y, ref, f"N={N} K={K} G={group} B={B}")


def test_tile_stream_offset_headers_take_another_kernel():
    """Header arrays one entry past an 8-byte boundary: the product runs on
    another kernel (the streaming 16-row kernel) and matches."""
    device()
    N, K, G, B = 2085, 4096, 128, 8
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    c, s, z = oracle.quantize(W, G, 4)

    def offset_copy(a):
        flat = torch.zeros(a.size + 8, dtype=torch.float16, device=device())
        flat[1:1 + a.size] = to_dev(a.reshape(-1))
        return flat[1:1 + a.size].view(a.shape)

    note("tile-stream offset headers")
    Y = wq.gemm(to_dev(X), to_dev(c), offset_copy(s), offset_copy(z), N=N, K=K, group=G, bits=4, path="mfma")
    assert_close(Y, oracle.gemm(X, c, s, z, N, K, G, 4), "offset headers")


def test_tile_stream_repeat_is_bitwise_equal():
    """The waves' sums are added in a fixed order: two calls agree bit for bit."""
    device()
    N, K, G = 4096, 8192, 128
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = to_dev(rng.standard_normal((16, K)).astype(np.float16))
    c, s, z = (to_dev(a) for a in oracle.quantize(W, G, 4))
    for B in (8, 16):
        note(f"tile-stream repeat B={B}")
        a = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=G, bits=4, path="mfma")
        b = wq.gemm(X[:B].contiguous(), c, s, z, N=N, K=K, group=G, bits=4, path="mfma")
        assert torch.equal(a, b)


def test_tile_stream_on_7b_rows_all_outputs():
    """The first 7360 rows of the 7B-class up-projection (K = 4096, 0.1 %
    outliers): 460 tiles, just under 1.8 per compute unit, so the tile-stream
    kernel takes B = 5 .. 16; every output against the oracle."""
    device()
    name = "mlp7b_up_k4096_n11008_g128"
    W, _ = wq_inputs.workload_arrays(name)
    W = np.ascontiguousarray(W[:7360])
    N, K = W.shape
    c, s, z = wq.quantize_pack(to_dev(W), 128, 4)
    cn, sn, zn = (t.cpu().numpy() for t in (c, s, z))
    Xb = np.random.default_rng(7).standard_normal((16, K)).astype(np.float16)
    for B in (8, 16):
        note(f"tile-stream {name}[:7360] B={B}")
        Y = wq.gemm(to_dev(Xb[:B]), c, s, z, N=N, K=K, group=128, bits=4, path="mfma")
        assert_close(Y, oracle.gemm(Xb[:B], cn, sn, zn, N, K, 128, 4), f"{name}[:7360] B={B}")
