"""GPU parity of the matrix-core kernels on the cases their tiling makes special.

The small-batch matrix-core kernel (3 <= B <= 32) keeps a K-slice of X in
LDS, so these tests cover: K that is not a multiple of the slice (rounds past
K inside the last slice), several slices added in slice order, each way of
reading group headers (one group per 128-k round, several rounds per group,
one group per row), rows not a multiple of the 16-row tile, and groups whose
zero point lies far outside the code range.  They also check that the split-K
workspace, cached per (device, stream), gives identical results when reused,
grown, and used from two streams.
"""

import numpy as np
import pytest

import oracle
from edge_groups import crafted_groups
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def packed(W, group, bits):
    c, s, z = oracle.quantize(W, group, bits)
    return (c, s, z), (to_dev(c), to_dev(s), to_dev(z))


# K values: 35 and 86 rounds of 128 k (not multiples of the 8-round ring turn),
# 64 rounds (two slices at B > 8), 128 rounds (several slices at any B).
@pytest.mark.parametrize("K,group,bits", [(4480, 128, 4), (11008, 128, 4), (8192, 256, 4),
                                          (16384, 128, 4), (4480, 4480, 8), (11008, 64, 8),
                                          (4096, 512, 8)])
@pytest.mark.parametrize("B", [3, 8, 9, 16, 17, 32])
def test_ragged_slices_and_header_modes(K, group, bits, B):
    device()
    rng = np.random.default_rng(K + 7 * B + bits)
    N = 61
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"matrix-core N={N} K={K} G={group} b={bits} B={B}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=group, bits=bits, path="mfma")
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), f"K={K} G={group} B={B}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("B", [4, 16, 24, 40])
def test_extreme_groups(bits, B):
    """Crafted groups (saturated zero points, subnormal and +-65504 values,
    constant groups) stacked into rows: every operand stays finite."""
    device()
    G = 128 if bits == 4 else 64
    rows = crafted_groups(G, bits, seed=3)              # [R, G], one case per row
    R = rows.shape[0]
    W = np.tile(rows, (1, 8))                           # K = 8 groups per row
    K = W.shape[1]
    rng = np.random.default_rng(bits * 100 + B)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, G, bits)
    note(f"crafted groups R={R} K={K} G={G} b={bits} B={B}")
    Y = wq.gemm(to_dev(X), *dev, N=R, K=K, group=G, bits=bits, path="mfma")
    ref = oracle.gemm(X, *host, R, K, G, bits)
    y = Y.cpu().numpy().astype(np.float64)
    # Weight rows whose products exceed the fp16 range of Y are left out: their
    # reference is not representable in the output dtype.
    ok = np.all(np.abs(ref) < 60000, axis=0)
    assert ok.sum() >= R // 2
    assert_close(y[:, ok], ref[:, ok], "crafted")


def test_workspace_reuse_and_growth():
    """Repeated, smaller and larger split-K calls on one stream reuse the same
    workspace and agree bit for bit with the first call of each shape."""
    device()
    shapes = [(300, 16384, 16), (40, 16384, 5), (900, 16384, 16), (300, 16384, 16)]
    first = {}
    for N, K, B in shapes:
        W = (np.random.default_rng(N).standard_normal((N, K)) * 0.02).astype(np.float16)
        X = np.random.default_rng(B + N).standard_normal((B, K)).astype(np.float16)
        host, dev = packed(W, 128, 4)
        note(f"workspace N={N} K={K} B={B}")
        Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
        if (N, B) in first:
            assert np.array_equal(Y.view(np.uint16), first[(N, B)].view(np.uint16))
        else:
            assert_close(Y.astype(np.float64), oracle.gemm(X, *host, N, K, 128, 4), "workspace")
            first[(N, B)] = Y


def test_two_streams():
    """Split-K calls on two streams (own workspaces) match the same calls on
    the default stream."""
    device()
    N, K, B = 500, 16384, 12
    W = (np.random.default_rng(31).standard_normal((N, K)) * 0.02).astype(np.float16)
    X = np.random.default_rng(32).standard_normal((B, K)).astype(np.float16)
    _, dev = packed(W, 128, 4)
    Xd = to_dev(X)
    ref = wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma"))
    torch.cuda.synchronize()
    for y in outs:
        assert np.array_equal(y.cpu().numpy().view(np.uint16), ref.view(np.uint16))
