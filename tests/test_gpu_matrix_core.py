"""GPU parity of the matrix-core kernels on the cases their tiling makes special.

The small-batch matrix-core kernel (3 <= B <= 32) keeps a K-slice of X in
LDS, so these tests cover: K that is not a multiple of the slice (rounds past
K inside the last slice), several slices added in slice order, each way of
reading group headers (one group per 128-k round, several rounds per group,
one group per row), rows not a multiple of the 16-row tile, and groups whose
zero point lies far outside the code range, each with the caller's workspace
(split partials) and without one (plans that need none).  They also check that
one workspace reused across calls of different shapes, and separate
workspaces on two streams, give results identical to fresh ones.
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
@pytest.mark.parametrize("use_ws", [True, False])
def test_ragged_slices_and_header_modes(K, group, bits, B, use_ws):
    device()
    rng = np.random.default_rng(K + 7 * B + bits)
    N = 61
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"matrix-core N={N} K={K} G={group} b={bits} B={B} workspace={use_ws}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=group, bits=bits, path="mfma", use_workspace=use_ws)
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
    # Each kept row on its own, against what the kernels' arithmetic can lose:
    #   - the tiled kernel's fp16 dequantization of each weight, (512 + q/2)
    #     minus the fp16 (512 + z/2) times s: at most three fp16 roundings,
    #     under 2^-9 of |x w| per term, or 2^-25 |x| for a subnormal weight;
    #   - fp32 sums of terms offset by up to 1040 * s per code (the exact-code
    #     kernels subtract the offset after summing), 2^-24 of the running
    #     magnitude per addition over K terms;
    #   - one fp16 rounding of the output, 2^-11 |y| (2^-25 absolute below the
    #     normal range).
    # Rows whose outputs are small are then held to their own size, not to
    # 1e-2 of the largest output of the whole test.
    What = oracle.dequantize(*host, R, K, G, bits)
    Xa = np.abs(X.astype(np.float64))
    s_full = np.repeat(host[1].astype(np.float64), G, axis=1)          # [R, K] scale of each weight
    mag = Xa @ np.abs(What).T
    offs = Xa @ (1040.0 * s_full).T
    bound = (2.0**-9 * mag + 2.0**-25 * Xa.sum(axis=1)[:, None] + K * 2.0**-24 * (mag + offs)
             + 2.0**-11 * np.abs(ref) + 2.0**-25)
    err = np.abs(y - ref)
    bad = (err > bound)[:, ok]
    assert not bad.any(), f"per-row bound exceeded at {np.argwhere(bad)[:5]}: err {err[:, ok][bad][:5]}"


def test_workspace_reuse_across_shapes():
    """One caller workspace, sized for the largest call, serves repeated,
    smaller and larger split-K calls in stream order; each result is identical
    to the same call with a fresh workspace, and within tolerance of the
    oracle."""
    device()
    shapes = [(300, 16384, 16), (40, 16384, 5), (900, 16384, 16), (300, 16384, 16), (4096, 11008, 40)]
    need = max(wq.gemm_workspace_bytes(B, K, N, 128, 4, "mfma") for N, K, B in shapes)
    assert need > 0
    shared = torch.empty(need, dtype=torch.uint8, device=device())
    shared.fill_(0xA5)                               # contents on entry do not matter
    for N, K, B in shapes:
        W = (np.random.default_rng(N).standard_normal((N, K)) * 0.02).astype(np.float16)
        X = np.random.default_rng(B + N).standard_normal((B, K)).astype(np.float16)
        host, dev = packed(W, 128, 4)
        note(f"workspace reuse N={N} K={K} B={B}")
        Xd = to_dev(X)
        Y = wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma", workspace=shared).cpu().numpy()
        fresh = wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
        assert np.array_equal(Y.view(np.uint16), fresh.view(np.uint16))
        assert_close(Y.astype(np.float64), oracle.gemm(X, *host, N, K, 128, 4), "workspace")


def test_undersized_workspace_raises():
    device()
    N, K, B = 300, 16384, 16
    need = wq.gemm_workspace_bytes(B, K, N, 128, 4, "mfma")
    assert need > 0
    W = (np.random.default_rng(5).standard_normal((N, K)) * 0.02).astype(np.float16)
    _, dev = packed(W, 128, 4)
    Xd = to_dev(np.ones((B, K), np.float16))
    small = torch.empty(need - 256, dtype=torch.uint8, device=device())
    with pytest.raises(ValueError):
        wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma", workspace=small)


def test_two_streams():
    """Split-K calls on two streams, each with its own workspace, match the
    same call on the default stream bit for bit."""
    device()
    N, K, B = 500, 16384, 12
    W = (np.random.default_rng(31).standard_normal((N, K)) * 0.02).astype(np.float16)
    X = np.random.default_rng(32).standard_normal((B, K)).astype(np.float16)
    _, dev = packed(W, 128, 4)
    Xd = to_dev(X)
    ref = wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
    need = wq.gemm_workspace_bytes(B, K, N, 128, 4, "mfma")
    assert need > 0
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws = [torch.empty(need, dtype=torch.uint8, device=device()) for _ in range(2)]
    torch.cuda.synchronize()
    outs = []
    for s, w in zip((s1, s2), ws):
        with torch.cuda.stream(s):
            outs.append(wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=4, path="mfma", workspace=w))
    torch.cuda.synchronize()
    for y in outs:
        assert np.array_equal(y.cpu().numpy().view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("N,K,B", [(8192, 1024, 256), (4100, 1024, 500), (12000, 512, 160)])
def test_tiled_128_row_tiles_past_the_ridge(N, K, B):
    """Past 64 batch columns, matrices whose 128-row tiles give one to two
    blocks per compute unit take two 16-row tiles per wave (ragged N and B,
    K-splits added in order); every output against the oracle."""
    device()
    rng = np.random.default_rng(N + B)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, 128, 4)
    note(f"tiled 128-row N={N} K={K} B={B}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=128, bits=4, path="mfma")
    assert_close(Y, oracle.gemm(X, *host, N, K, 128, 4), f"N={N} K={K} B={B}")
