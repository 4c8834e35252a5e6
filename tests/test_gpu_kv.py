"""GPU parity of the int4 KV cache: quantize-on-append bit-exact with the
oracle, and decode attention within the product tolerance of the float64
oracle ("What actually happens when you quantize a KV cache").

Cases: crafted K/V blocks (ties, constant and subnormal groups, +-65504, a hot
channel); heads holding 0, 1, 127, 128, 129, ... 4096 tokens (empty cache,
residual only, whole blocks, both), which reach one split per head, many
splits, and empty splits; lengths past the cache's capacity (clamped) and
negative; and the 7B-class decode configuration (1024 heads x 4096 tokens)
on sampled heads.
"""

import numpy as np
import pytest

import oracle
import oracle.kv as okv
from edge_groups import crafted_groups
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = G = 128


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def draw_kv(rng, T):
    K = rng.standard_normal((T, D))
    K[:, 3] *= 8.0                                  # a hot key channel
    V = rng.standard_normal((T, D))
    return K.astype(np.float16), V.astype(np.float16)


def build(heads_kv, max_blocks):
    """GPU cache from per-head fp16 K, V [T_h, D]: full blocks through
    wq_kv_quantize_block, the rest copied into the residual window."""
    H = len(heads_kv)
    cache = wq.KVCache(H, max_blocks)
    nblk = [min(len(K) // G, max_blocks) for K, _ in heads_kv]
    for j in range(max(nblk) if nblk else 0):
        Kb = np.zeros((H, G, D), np.float16)
        Vb = np.zeros((H, G, D), np.float16)
        for h, (K, V) in enumerate(heads_kv):
            if j < nblk[h]:
                Kb[h], Vb[h] = K[j * G:(j + 1) * G], V[j * G:(j + 1) * G]
        wq.kv_quantize_block(to_dev(Kb), to_dev(Vb), cache, j)
    for h, (K, V) in enumerate(heads_kv):
        r = len(K) - nblk[h] * G
        if 0 < r < G:
            cache.kres[h, :r] = to_dev(K[nblk[h] * G:])
            cache.vres[h, :r] = to_dev(V[nblk[h] * G:])
    return cache, nblk


def oracle_out(q, K, V, nblk):
    blocks = [okv.quantize_block(K[j * G:(j + 1) * G], V[j * G:(j + 1) * G]) for j in range(nblk)]
    return okv.decode_head(q, blocks, K[nblk * G:], V[nblk * G:])


def test_quantize_block_bit_exact():
    device()
    rng = np.random.default_rng(1)
    cols = crafted_groups(G, 4, seed=5)            # rows of 128 values, one corner case each
    heads = []
    for h in range(6):
        K, V = draw_kv(rng, G)
        if h < 3:
            n = min(D, cols.shape[0])
            K[:, :n] = cols[(np.arange(n) + 7 * h) % cols.shape[0]].T   # crafted K channels
            V[:n, :] = cols[(np.arange(n) + 5 * h) % cols.shape[0]]      # crafted V tokens
        heads.append((K, V))
    note("kv quantize block: 6 heads (3 crafted)")
    cache, _ = build(heads, 2)
    torch.cuda.synchronize()
    for h, (K, V) in enumerate(heads):
        blk = okv.quantize_block(K, V)
        assert np.array_equal(cache.kcodes[h, 0].cpu().numpy(), blk["kcodes"]), h
        assert np.array_equal(_u16(cache.kscales[h, 0]), blk["ks"].view(np.uint16)), h
        assert np.array_equal(_u16(cache.kzeros[h, 0]), blk["kz"].view(np.uint16)), h
        assert np.array_equal(cache.vcodes[h, 0].cpu().numpy(), blk["vcodes"]), h
        assert np.array_equal(_u16(cache.vscales[h, :G]), blk["vs"].view(np.uint16)), h
        assert np.array_equal(_u16(cache.vzeros[h, :G]), blk["vz"].view(np.uint16)), h
    # Block 1 was never written for any head: untouched.
    assert not cache.kcodes[:, 1].any() and not cache.vcodes[:, 1].any()


def test_quantize_block_bit_exact_many_heads():
    """256 heads at the benchmark's distribution (N(0, 1), one hot K channel),
    written into block 3 of 5: every code and header bit for bit, and the
    other blocks untouched.  Each head's 16 384 values go through the fp32
    quotient estimate, and the waves with a value near a half-integer through
    the exact decision."""
    device()
    H, nb, j = 256, 5, 3
    rng = np.random.default_rng(17)
    Kb = np.empty((H, G, D), np.float16)
    Vb = np.empty((H, G, D), np.float16)
    for h in range(H):
        Kb[h], Vb[h] = draw_kv(rng, G)
    note("kv quantize block: 256 heads, block 3")
    cache = wq.KVCache(H, nb)
    wq.kv_quantize_block(to_dev(Kb), to_dev(Vb), cache, j)
    torch.cuda.synchronize()
    kc, vc = cache.kcodes[:, j].cpu().numpy(), cache.vcodes[:, j].cpu().numpy()
    ks, kz = _u16(cache.kscales[:, j]), _u16(cache.kzeros[:, j])
    vs, vz = _u16(cache.vscales[:, j * G:(j + 1) * G]), _u16(cache.vzeros[:, j * G:(j + 1) * G])
    for h in range(H):
        blk = okv.quantize_block(Kb[h], Vb[h])
        assert np.array_equal(kc[h], blk["kcodes"]), h
        assert np.array_equal(ks[h], blk["ks"].view(np.uint16)), h
        assert np.array_equal(kz[h], blk["kz"].view(np.uint16)), h
        assert np.array_equal(vc[h], blk["vcodes"]), h
        assert np.array_equal(vs[h], blk["vs"].view(np.uint16)), h
        assert np.array_equal(vz[h], blk["vz"].view(np.uint16)), h
    others = [b for b in range(nb) if b != j]
    assert not cache.kcodes[:, others].any() and not cache.vcodes[:, others].any()


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("max_blocks", [32, 1])
def test_attention_ragged_lengths(max_blocks, use_ws):
    """max_blocks 32: many splits per head (some empty) with a workspace, one
    workgroup per head without; max_blocks 1: one split."""
    device()
    rng = np.random.default_rng(2 + max_blocks)
    lens = [0, 1, 5, 127, 128, 129, 255, 256, 300, 1000, 4096]
    if max_blocks == 1:
        lens = [0, 1, 127, 128, 129, 200, 255]
    heads = [draw_kv(rng, T) for T in lens]
    q = rng.standard_normal((len(lens), D)).astype(np.float16)
    note(f"kv attention lens={lens} max_blocks={max_blocks} workspace={use_ws}")
    cache, nblk = build(heads, max_blocks)
    out = wq.kv_attention(to_dev(q), cache, to_dev(np.array(lens, np.int32)), use_workspace=use_ws)
    ref = np.stack([oracle_out(q[h], K, V, nblk[h]) for h, (K, V) in enumerate(heads)])
    got = out.cpu().numpy().astype(np.float64)
    assert not got[0].any()                         # empty cache -> zeros
    assert_close(got, ref, "ragged")
    again = wq.kv_attention(to_dev(q), cache, to_dev(np.array(lens, np.int32)),
                            use_workspace=use_ws).cpu().numpy()
    assert np.array_equal(again.view(np.uint16), out.cpu().numpy().view(np.uint16))


def test_lengths_are_clamped():
    device()
    rng = np.random.default_rng(9)
    heads = [draw_kv(rng, 2 * G + 127), draw_kv(rng, G)]
    cache, nblk = build(heads, 2)
    q = rng.standard_normal((2, D)).astype(np.float16)
    # Head 0 claims far more tokens than the cache holds; head 1 a negative count.
    out = wq.kv_attention(to_dev(q), cache, to_dev(np.array([10 ** 6, -5], np.int32)))
    got = out.cpu().numpy().astype(np.float64)
    K, V = heads[0]
    assert_close(got[:1], oracle_out(q[0], K, V, 2)[None], "clamped to capacity")
    assert not got[1].any()


def test_decode_7b_configuration_sampled():
    """32 layers x 32 heads = 1024 heads, 4096 tokens each (the page's receipt
    configuration), inputs drawn on the GPU; sampled heads against the oracle."""
    device()
    H, T = 1024, 4096
    nb = T // G
    gen = torch.Generator(device="cuda").manual_seed(7)
    cache = wq.KVCache(H, nb)
    sample = [0, 1, 511, 1023]
    hostK = {h: [] for h in sample}
    hostV = {h: [] for h in sample}
    note("kv 7B configuration: building 32 blocks x 1024 heads")
    for j in range(nb):
        Kb = torch.randn((H, G, D), generator=gen, device="cuda")
        Kb[:, :, 3] *= 8.0
        Kb = Kb.half()
        Vb = torch.randn((H, G, D), generator=gen, device="cuda").half()
        wq.kv_quantize_block(Kb, Vb, cache, j)
        for h in sample:
            hostK[h].append(Kb[h].cpu().numpy())
            hostV[h].append(Vb[h].cpu().numpy())
    q = torch.randn((H, D), generator=gen, device="cuda").half()
    lens = torch.full((H,), T, dtype=torch.int32, device="cuda")
    out = wq.kv_attention(q, cache, lens).cpu().numpy().astype(np.float64)
    qh = q.cpu().numpy()
    for h in sample:
        K = np.concatenate(hostK[h])
        V = np.concatenate(hostV[h])
        ref = oracle_out(qh[h], K, V, nb)
        assert_close(out[h:h + 1], ref[None], f"head {h}")
