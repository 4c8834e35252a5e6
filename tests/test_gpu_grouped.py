"""GPU parity of wq_gemm_grouped: every item's output is bit-identical to a
separate wq_gemm call on the same inputs, and matches the CPU oracle.

Grouping puts the X-resident products of one batch size and bit width into
shared launches (up to eight per launch, one launch per group-header layout,
one reduction launch); everything else runs as single calls.  The cases mix
all of these: several header layouts in one call, more than eight grouped
products, batch sizes that take the GEMV and the tiled kernel, and a whole
7B-class decode layer at B = 32.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def make_item(rng, B, N, K, group, bits, host=False):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    Wd = to_dev(W)
    c, s, z = wq.quantize_pack(Wd, group=group, bits=bits)
    item = (to_dev(X), c, s, z, N, K, group, bits)
    if host:
        return item, (X, W)
    return item


def single(item):
    X, c, s, z, N, K, group, bits = item
    return wq.gemm(X, c, s, z, N=N, K=K, group=group, bits=bits)


def assert_bitwise(outs, items):
    torch.cuda.synchronize()
    for i, (y, it) in enumerate(zip(outs, items)):
        ref = single(it)
        torch.cuda.synchronize()
        a = y.cpu().numpy().view(np.uint16)
        b = ref.cpu().numpy().view(np.uint16)
        assert np.array_equal(a, b), f"item {i}: B={it[0].shape[0]} N={it[4]} K={it[5]} G={it[6]} b={it[7]}"


def test_mixed_items_match_single_calls():
    """Header layouts (one group per round, several rounds per group, one
    group per row), GEMV and tiled items, two bit widths, in one call."""
    device()
    rng = np.random.default_rng(21)
    specs = [
        (16, 300, 4096, 128, 4),    # x-resident, 8 groups per 128-bit load
        (16, 200, 4096, 256, 4),    # x-resident, a group spans two rounds
        (16, 150, 4480, 128, 4),    # x-resident, 35 groups: one load per round
        (16, 100, 2048, 2048, 4),   # x-resident, one group per row
        (1, 333, 8192, 128, 4),     # GEMV (one-row kernel)
        (40, 130, 2048, 128, 4),    # tiled
        (16, 120, 2048, 64, 8),     # 8-bit: another (B, bits) group
        (16, 257, 4096, 128, 4),    # back to the first group
        (5, 90, 1024, 128, 4),      # x-resident, 8-column tile
        (24, 210, 4096, 128, 4),    # x-resident, two column blocks per wave
    ]
    items = [make_item(rng, *sp) for sp in specs]
    note(f"grouped mixed: {len(items)} items")
    outs = wq.gemm_grouped(items)
    assert_bitwise(outs, items)


def test_more_than_eight_grouped_products():
    """Eleven products of one kind take two grouped launches."""
    device()
    rng = np.random.default_rng(22)
    items = [make_item(rng, 12, 64 + 37 * i, 2048 + 1024 * (i % 3), 128, 4) for i in range(11)]
    note("grouped: 11 products at B=12")
    outs = wq.gemm_grouped(items)
    assert_bitwise(outs, items)


@pytest.mark.parametrize("bits,group", [(4, 128), (8, None)])
def test_decode_layer_at_b32(bits, group):
    """The seven matrices of a 7B-class layer (int4 g128 or 8-bit per-channel)
    at B = 32 in one call; four of them are also checked against the oracle
    on sampled rows."""
    device()
    rng = np.random.default_rng(23 + bits)
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    items, hosts = [], []
    for N, K in shapes:
        G = group if group else K
        it, h = make_item(rng, 32, N, K, G, bits, host=True)
        items.append(it)
        hosts.append(h)
    note(f"grouped decode layer b={bits}")
    outs = wq.gemm_grouped(items)
    assert_bitwise(outs, items)
    for idx in (0, 3, 4, 6):
        X, W = hosts[idx]
        N, K = shapes[idx]
        G = group if group else K
        # Rows are independent: the oracle quantizes and multiplies only the
        # sampled ones.
        rows = np.sort(rng.choice(N, 48, replace=False))
        c, s, z = oracle.quantize(W[rows], G, bits)
        ref = oracle.gemm(X, c, s, z, len(rows), K, G, bits)
        y = outs[idx].cpu().numpy().astype(np.float64)[:, rows]
        assert_close(y, ref, f"layer item {idx}")


def test_empty_and_noop_items():
    device()
    rng = np.random.default_rng(24)
    assert wq.gemm_grouped([]) == []
    it = make_item(rng, 8, 100, 2048, 128, 4)
    X, c, s, z, N, K, G, b = it
    empty = (X[:0], c, s, z, N, K, G, b)
    outs = wq.gemm_grouped([empty, it])
    assert outs[0].shape == (0, N)
    assert_bitwise(outs[1:], [it])
