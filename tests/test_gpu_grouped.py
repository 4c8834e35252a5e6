"""GPU parity of wq_gemm_grouped: every item matches the CPU oracle and a
separate wq_gemm call on the same inputs (to the product tolerance: grouped
launches slice K differently), and repeated grouped calls agree bit for bit.

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


def assert_matches_single(outs, items):
    """Each grouped output is within the product tolerance of a single call,
    and a second grouped call reproduces every output bit for bit."""
    torch.cuda.synchronize()
    again = wq.gemm_grouped(items)
    torch.cuda.synchronize()
    for i, (y, y2, it) in enumerate(zip(outs, again, items)):
        what = f"item {i}: B={it[0].shape[0]} N={it[4]} K={it[5]} G={it[6]} b={it[7]}"
        a = y.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), y2.cpu().numpy().view(np.uint16)), what
        ref = single(it).cpu().numpy().astype(np.float64)
        if ref.size:
            assert_close(a.astype(np.float64), ref, what)


def assert_matches_oracle(outs, items, hosts, rng, nrows=40):
    """Sampled rows of every item against the oracle (rows are independent,
    so the oracle quantizes and multiplies only those)."""
    for i, (y, it, (X, W)) in enumerate(zip(outs, items, hosts)):
        N, K, G, bits = it[4], it[5], it[6], it[7]
        rows = np.sort(rng.choice(N, min(nrows, N), replace=False))
        c, s, z = oracle.quantize(W[rows], G, bits)
        ref = oracle.gemm(X, c, s, z, len(rows), K, G, bits)
        assert_close(y.cpu().numpy().astype(np.float64)[:, rows], ref, f"item {i} vs oracle")


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
    made = [make_item(rng, *sp, host=True) for sp in specs]
    items = [m[0] for m in made]
    note(f"grouped mixed: {len(items)} items")
    outs = wq.gemm_grouped(items)
    assert_matches_single(outs, items)
    assert_matches_oracle(outs, items, [m[1] for m in made], rng)
    # Without a workspace every product takes a plan with no K-split partials.
    note(f"grouped mixed without workspace: {len(items)} items")
    bare = wq.gemm_grouped(items, use_workspace=False)
    torch.cuda.synchronize()
    assert_matches_oracle(bare, items, [m[1] for m in made], rng)


def test_more_than_eight_grouped_products():
    """Eleven products of one kind take two grouped launches."""
    device()
    rng = np.random.default_rng(22)
    made = [make_item(rng, 12, 64 + 37 * i, 2048 + 1024 * (i % 3), 128, 4, host=True) for i in range(11)]
    items = [m[0] for m in made]
    note("grouped: 11 products at B=12")
    outs = wq.gemm_grouped(items)
    assert_matches_single(outs, items)
    assert_matches_oracle(outs, items, [m[1] for m in made], rng)


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("bits,group", [(4, 128), (8, None)])
def test_decode_layer_at_b32(bits, group, use_ws):
    """The seven matrices of a 7B-class layer (int4 g128 or 8-bit per-channel)
    at B = 32 in one call, each checked against the oracle on sampled rows."""
    device()
    rng = np.random.default_rng(23 + bits)
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    items, hosts = [], []
    for N, K in shapes:
        G = group if group else K
        it, h = make_item(rng, 32, N, K, G, bits, host=True)
        items.append(it)
        hosts.append(h)
    note(f"grouped decode layer b={bits} workspace={use_ws}")
    outs = wq.gemm_grouped(items, use_workspace=use_ws)
    if use_ws:
        assert_matches_single(outs, items)
    assert_matches_oracle(outs, items, hosts, rng, nrows=48)


def test_empty_and_noop_items():
    device()
    rng = np.random.default_rng(24)
    assert wq.gemm_grouped([]) == []
    it = make_item(rng, 8, 100, 2048, 128, 4)
    X, c, s, z, N, K, G, b = it
    empty = (X[:0], c, s, z, N, K, G, b)
    outs = wq.gemm_grouped([empty, it])
    assert outs[0].shape == (0, N)
    torch.cuda.synchronize()
    # A lone x-resident product keeps the single-call plan: bit-identical.
    assert np.array_equal(outs[1].cpu().numpy().view(np.uint16), single(it).cpu().numpy().view(np.uint16))
