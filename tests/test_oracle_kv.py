"""Pins of the KV-cache attention oracle (CPU only).

"What actually happens when you quantize a KV cache": the codec of §3-§4
applied per channel to K and per token to V (§7 "axis choice"), the byte
receipt of §5-§6, and decode attention (§2).  The codec is checked element by
element against the exact-rational brute force, reading the codes from the
cache layout's definition; attention against a library softmax-attention on
a cache dequantized here from that same definition, and against closed forms.
"""

import numpy as np
import pytest

import bruteforce
from conftest import read_golden

F16 = np.float16


@pytest.fixture(scope="module")
def kv(oracle_mod):
    import oracle.kv as kvmod
    return kvmod


def nibble(row, i):
    return (int(row[i // 2]) >> (4 * (i % 2))) & 0xF


def _blocks(rng, nblk, G=128, D=128, hot=3):
    out = []
    for _ in range(nblk):
        K = rng.standard_normal((G, D)) * 0.5
        K[:, hot] *= 10.0                      # a hot key channel, as §7 describes
        V = rng.standard_normal((G, D)) * 0.5
        out.append((K.astype(F16), V.astype(F16)))
    return out


@pytest.mark.parametrize("G,D", [(8, 8), (16, 8), (8, 32)])
def test_block_codec_matches_bruteforce(kv, G, D):
    rng = np.random.default_rng(G * 100 + D)
    K = (rng.standard_normal((G, D)) * 0.3).astype(F16)
    K[:, 1] *= 8
    V = (rng.standard_normal((G, D)) * 0.3).astype(F16)
    blk = kv.quantize_block(K, V)
    kb = K.view(np.uint16)
    vb = V.view(np.uint16)
    for d in range(D):                          # K: one group per channel
        q, s, z = bruteforce.quantize_group([int(v) for v in kb[:, d]], 4)
        assert blk["ks"].view(np.uint16)[d] == s and blk["kz"].view(np.uint16)[d] == z
        for t in range(G):
            assert nibble(blk["kcodes"][t], d) == q[t]
    for t in range(G):                          # V: one group per token
        q, s, z = bruteforce.quantize_group([int(v) for v in vb[t, :]], 4)
        assert blk["vs"].view(np.uint16)[t] == s and blk["vz"].view(np.uint16)[t] == z
        for d in range(D):
            assert nibble(blk["vcodes"][d], t) == q[d]


def _dequant_here(blk):
    """Dequantize from the layout definition, element by element."""
    G, D = blk["vs"].shape[0], blk["ks"].shape[0]
    K = np.empty((G, D))
    V = np.empty((G, D))
    for t in range(G):
        for d in range(D):
            K[t, d] = (nibble(blk["kcodes"][t], d) - float(blk["kz"][d])) * float(blk["ks"][d])
            V[t, d] = (nibble(blk["vcodes"][d], t) - float(blk["vz"][t])) * float(blk["vs"][t])
    return K, V


@pytest.mark.parametrize("nblk,res", [(0, 37), (1, 0), (2, 5), (3, 127)])
def test_attention_matches_library_softmax(kv, nblk, res):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(nblk * 10 + res)
    D = 128
    blocks = [kv.quantize_block(K, V) for K, V in _blocks(rng, nblk)]
    kr = (rng.standard_normal((res, D)) * 0.5).astype(F16)
    vr = (rng.standard_normal((res, D)) * 0.5).astype(F16)
    q = (rng.standard_normal(D)).astype(F16)
    out = kv.decode_head(q, blocks, kr, vr)
    Ks = [_dequant_here(b)[0] for b in blocks] + [kr.astype(np.float64)]
    Vs = [_dequant_here(b)[1] for b in blocks] + [vr.astype(np.float64)]
    K = torch.from_numpy(np.concatenate(Ks))[None, None]
    V = torch.from_numpy(np.concatenate(Vs))[None, None]
    Q = torch.from_numpy(q.astype(np.float64))[None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[0, 0, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms(kv):
    rng = np.random.default_rng(3)
    D = 128
    blocks = [kv.quantize_block(K, V) for K, V in _blocks(rng, 2)]
    Ks, Vs = zip(*[_dequant_here(b) for b in blocks])
    # q = 0: every score is 0, the output is the plain mean of V.
    out = kv.decode_head(np.zeros(D, F16), blocks, np.zeros((0, D), F16), np.zeros((0, D), F16))
    assert np.allclose(out, np.concatenate(Vs).mean(0), rtol=0, atol=1e-12)
    # One key aligned with q and far larger than the rest: its value wins.
    q = np.zeros(D, F16)
    q[5] = 1.0
    kr = np.zeros((3, D), F16)
    kr[1, 5] = 4096.0
    vr = (rng.standard_normal((3, D))).astype(F16)
    out = kv.decode_head(q, blocks, kr, vr)
    assert np.allclose(out, vr[1].astype(np.float64), rtol=0, atol=1e-9)
    # An empty cache gives zeros.
    assert not np.any(kv.attend(np.ones(D), np.zeros((0, D)), np.zeros((0, D)), 1.0))


def test_receipt_matches_page(kv):
    g = read_golden("kvq_receipt.txt")
    L, H, D, G = (int(g[k]) for k in ("layers", "kv_heads", "head_dim", "group"))
    heads = L * H
    assert 2 * D * 2 * heads == int(g["fp16_bytes_per_token"])
    assert 2 * D * 4 // 8 * heads == int(g["int4_element_bytes_per_token"])
    assert 2 * heads * D // G == int(g["header_groups_per_token"])
    assert 4 * int(g["header_groups_per_token"]) == int(g["header_bytes_per_token"])
    per_token = kv.cache_bytes_per_token(D, G) * heads
    assert per_token == int(g["int4_total_kib_per_token"]) * 1024
    T = int(g["context"])
    assert round(T * 2 * D * 2 * heads / 2 ** 30, 1) == float(g["fp16_sequence_gib"])
    assert T * per_token / 2 ** 20 == float(g["int4_sequence_mib"])
    bw = float(g["bandwidth_tb_s"]) * 1e12
    assert round(T * 2 * D * 2 * heads / bw * 1e3, 2) == float(g["fp16_stream_ms"])
    assert round(T * per_token / bw * 1e3, 2) == float(g["int4_stream_ms"])
    assert per_token * 8 / (2 * D * heads) == float(g["effective_bits"])
    assert round(2 * D * 2 * heads / per_token, 2) == float(g["ratio"])
