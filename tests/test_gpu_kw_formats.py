"""GPU parity of 2- and 3-bit codes, of the float-offset variant at 2, 3 and
4 bits, and of NF4 codes (blocks of 64) on the K-split-wave matrix-core kernel (2 <= B <= 32, group 128,
K = 2048, 4096 or 8192, at least 1.8 16-row tiles per compute unit;
wq_gemm_kw.hip) against the CPU oracle.

The codes are unpacked as exact fp16 integers E + q, each operand slot with
its own exponent E (2 bits: 1024, 256, 64, 16; 3 bits: 1024, 128, 16, 1024),
E is subtracted exactly in fp16, and the group header is applied once per
128-k round in fp32; NF4 codes become fp16 level pairs through an LDS table
and are scaled in fp16 (level * s, rounded once)
("Quantization & inference optimisation", section "Quantization": the integer
and the group's endpoints give back the weight; its error table covers 8, 4,
3 and 2 bits).  What the shapes exercise:
  - K = 2048, 4096, 8192 (one, two or four two-round steps per wave);
  - 2 to 8 tiles per block, a partial last tile (N % 16 != 0);
  - one and two 16-row batch blocks, batch rows past B read as zeros;
  - integer zero points from the asymmetric and both symmetric schemes, and
    float offsets (x_hat = q s + m);
  - the routing: B = 1 and B > 32 stay on the bit-stream GEMV.
Every output is compared, except on the 70B-class matrix for the float
offsets (whose oracle dequantizes the whole matrix in float64): sampled rows
there.
"""

import numpy as np
import pytest

import oracle
import oracle.nf4 as onf4
import wq_inputs
from gpu_util import assert_close, device, note, to_dev, torch

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K, batches)
    (8192, 8192, (2, 16, 32)),           # 2 tiles per block
    (7376, 2048, (2, 32)),               # 461 tiles (the fewest taken), one step per wave
    (11990, 4096, (5, 17)),              # 3 tiles per block, partial last tile
    (12305, 2048, (2, 5, 16, 17, 32)),   # 4 tiles per block, partial last tile
    (16400, 4096, (3, 16, 24)),          # 5 tiles per block
    (12400, 8192, (2, 16, 32)),          # 4 tiles per block, four steps per wave
]


def _draw(N, K, Bmax, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((Bmax, K)).astype(np.float16)
    return W, X


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("N,K,batches", SHAPES)
def test_low_bit_codes_all_outputs(bits, N, K, batches):
    device()
    W, X = _draw(N, K, max(batches), N + 17 * K + bits)
    c, s, z = oracle.quantize(W, 128, bits)
    dev = [to_dev(a) for a in (c, s, z)]
    for B in batches:
        note(f"kw formats b={bits} N={N} K={K} B={B}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=128, bits=bits, path="mfma")
        assert_close(Y, oracle.gemm(X[:B], c, s, z, N, K, 128, bits), f"b={bits} N={N} K={K} B={B}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("scheme", ["sym", "sym_tensor"])
def test_low_bit_symmetric_schemes(bits, scheme):
    """Symmetric codes carry 2^(b-1) as every group's zero point; per tensor,
    most codes sit next to it (the hardest case for the sums' precision)."""
    device()
    N, K = 12305, 4096
    W, X = _draw(N, K, 16, 31 + bits)
    c, s, z = oracle.quantize(W, 128, bits, scheme=scheme)
    for B in (4, 16):
        note(f"kw formats {scheme} b={bits} B={B}")
        Y = wq.gemm(to_dev(X[:B]), to_dev(c), to_dev(s), to_dev(z), N=N, K=K, group=128, bits=bits)
        assert_close(Y, oracle.gemm(X[:B], c, s, z, N, K, 128, bits), f"{scheme} b={bits} B={B}")


@pytest.mark.parametrize("bits", [2, 3])
def test_low_bit_routing_edges(bits):
    """B = 1 and B = 33 run on the bit-stream GEMV; both match the oracle, and
    the GEMV forced at B = 16 matches the matrix-core result's tolerance."""
    device()
    N, K = 12305, 2048
    W, X = _draw(N, K, 33, 47 + bits)
    c, s, z = oracle.quantize(W, 128, bits)
    dev = [to_dev(a) for a in (c, s, z)]
    for B, path in ((1, "auto"), (33, "auto"), (16, "gemv")):
        note(f"kw formats routing b={bits} B={B} path={path}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=128, bits=bits, path=path)
        assert_close(Y, oracle.gemm(X[:B], c, s, z, N, K, 128, bits), f"b={bits} B={B} {path}")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("B", [16, 32])
def test_low_bit_on_the_70b_matrix_all_rows(bits, B):
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    Xb = np.random.default_rng(5).standard_normal((B, K)).astype(np.float16)
    c, s, z = wq.quantize_pack(to_dev(W), 128, bits)
    cn, sn, zn = (t.cpu().numpy() for t in (c, s, z))
    note(f"kw formats {name} b={bits} B={B}")
    Y = wq.gemm(to_dev(Xb), c, s, z, N=N, K=K, group=128, bits=bits)
    assert_close(Y, oracle.gemm(Xb, cn, sn, zn, N, K, 128, bits), f"{name} b={bits} B={B}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,K,batches", [(12305, 2048, (2, 16, 17, 32)), (16400, 4096, (9,)),
                                         (7400, 4096, (3, 32))])
def test_float_offset_all_outputs(bits, N, K, batches):
    device()
    W, X = _draw(N, K, max(batches), 3 * N + K + bits)
    W[5, 3] = 0.7   # one outlier group
    c, s, m = oracle.quantize(W, 128, bits, scheme="offset")
    dev = [to_dev(a) for a in (c, s, m)]
    for B in batches:
        note(f"kw formats offset b={bits} N={N} K={K} B={B}")
        Y = wq.gemm_offset(to_dev(X[:B]), *dev, N=N, K=K, group=128, bits=bits)
        assert_close(Y, oracle.gemm_offset(X[:B], c, s, m, K, 128, bits), f"offset b={bits} N={N} K={K} B={B}")


@pytest.mark.parametrize("bits", [2, 4])
def test_float_offset_on_the_70b_matrix_sampled_rows(bits):
    """The 70B-class up-projection at B = 16 (the benchmark's table line):
    rows sampled across the whole matrix, every block's first and last tiles
    of the first and last blocks included."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    Xb = np.random.default_rng(8).standard_normal((16, K)).astype(np.float16)
    c, s, m = wq.quantize_pack(to_dev(W), 128, bits, scheme="offset")
    note(f"kw formats offset {name} b={bits}")
    Y = wq.gemm_offset(to_dev(Xb), c, s, m, N=N, K=K, group=128, bits=bits).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(N - 256, N),
                                     np.random.default_rng(9).choice(N, 512, replace=False)]))
    cn, sn, mn = (t.cpu().numpy()[rows] for t in (c, s, m))
    assert_close(Y[:, rows], oracle.gemm_offset(Xb, cn, sn, mn, K, 128, bits), f"offset {name} b={bits}")


@pytest.mark.parametrize("N,K,batches", [(12305, 2048, (2, 16, 17, 32)), (16400, 4096, (3, 16)),
                                         (12400, 8192, (9,)), (8192, 8192, (2, 32)), (11990, 4096, (16,))])
def test_nf4_all_outputs(N, K, batches):
    """NF4 ("Gör inference billig", the NF4 paragraph): sixteen normal-quantile
    levels, one absolute-maximum scale per block of 64."""
    device()
    W, X = _draw(N, K, max(batches), 5 * N + K)
    W[3, 7] = 0.6   # one outlier block
    c, s = onf4.quantize(W, 64)
    dc, ds = to_dev(c), to_dev(s)
    for B in batches:
        note(f"kw formats nf4 N={N} K={K} B={B}")
        Y = wq.gemm_nf4(to_dev(X[:B]), dc, ds, N=N, K=K, group=64)
        assert_close(Y, onf4.gemm(X[:B], c, s, K, 64), f"nf4 N={N} K={K} B={B}")


def test_nf4_routing_edges():
    """B = 1, B = 33 and blocks of 128 run on the NF4 GEMV; all match the oracle."""
    device()
    N, K = 12305, 2048
    W, X = _draw(N, K, 33, 71)
    for B, G in ((1, 64), (33, 64), (16, 128)):
        c, s = onf4.quantize(W, G)
        note(f"kw formats nf4 routing B={B} G={G}")
        Y = wq.gemm_nf4(to_dev(X[:B]), to_dev(c), to_dev(s), N=N, K=K, group=G)
        assert_close(Y, onf4.gemm(X[:B], c, s, K, G), f"nf4 B={B} G={G}")


def test_nf4_on_the_70b_matrix_sampled_rows():
    """The 70B-class up-projection at B = 16, quantized on the GPU: rows
    sampled across the whole matrix."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    Xb = np.random.default_rng(10).standard_normal((16, K)).astype(np.float16)
    c, s, _ = wq.quantize_pack(to_dev(W), 64, 4, scheme="nf4")
    note(f"kw formats nf4 {name}")
    Y = wq.gemm_nf4(to_dev(Xb), c, s, N=N, K=K, group=64).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(N - 256, N),
                                     np.random.default_rng(11).choice(N, 512, replace=False)]))
    assert_close(Y[:, rows], onf4.gemm(Xb, c.cpu().numpy()[rows], s.cpu().numpy()[rows], K, 64), f"nf4 {name}")


@pytest.mark.parametrize("bits,scheme,B", [(3, "offset", 3), (2, "offset", 3), (4, "offset", 3), (4, "asym", 5)])
def test_small_batch_two_tile_blocks_repeat_is_bitwise_equal(bits, scheme, B):
    """Blocks of two tiles at B = 3 and 5: the X rows past B of every slot read
    as zeros at once, so a slot refill that overtook the round's own LDS reads
    would change the result from call to call.  Ten calls agree bit for bit
    and match the oracle."""
    device()
    N, K = 7400, 4096
    W, X = _draw(N, K, B, 97 + bits)
    if scheme == "offset":
        c, s, m = oracle.quantize(W, 128, bits, scheme="offset")
        ref = oracle.gemm_offset(X, c, s, m, K, 128, bits)
        call = lambda: wq.gemm_offset(Xd, *dev, N=N, K=K, group=128, bits=bits)
    else:
        c, s, m = oracle.quantize(W, 128, bits)
        ref = oracle.gemm(X, c, s, m, N, K, 128, bits)
        call = lambda: wq.gemm(Xd, *dev, N=N, K=K, group=128, bits=bits, path="mfma")
    dev = [to_dev(a) for a in (c, s, m)]
    Xd = to_dev(X)
    note(f"kw formats repeat {scheme} b={bits} N={N} K={K} B={B}")
    first = call()
    assert_close(first, ref, f"repeat {scheme} b={bits}")
    for _ in range(9):
        assert torch.equal(call(), first)


def _offset_headers(a):
    """Device copy of a header array one entry past a 16-byte boundary."""
    flat = torch.zeros(a.size + 8, dtype=torch.float16, device=device())
    flat[1:1 + a.size] = to_dev(a.reshape(-1))
    return flat[1:1 + a.size].view(a.shape)


@pytest.mark.parametrize("fmt", ["int4", "int2", "int3", "offset", "nf4"])
def test_unaligned_headers_take_other_kernels(fmt):
    """Header arrays that are only 2-byte aligned (allowed by the interface)
    are not staged by the K-split-wave kernel's 16-byte loads: the shape
    (12305 x 2048, B = 16) then runs on another kernel, and matches the
    oracle and the aligned call's result."""
    device()
    N, K, B = 12305, 2048, 16
    W, X = _draw(N, K, B, 211)
    Xd = to_dev(X)
    note(f"kw formats unaligned headers {fmt}")
    if fmt == "nf4":
        c, s = onf4.quantize(W, 64)
        ref = onf4.gemm(X, c, s, K, 64)
        ya = wq.gemm_nf4(Xd, to_dev(c), to_dev(s), N=N, K=K, group=64)
        yu = wq.gemm_nf4(Xd, to_dev(c), _offset_headers(s), N=N, K=K, group=64)
    elif fmt == "offset":
        c, s, m = oracle.quantize(W, 128, 4, scheme="offset")
        ref = oracle.gemm_offset(X, c, s, m, K, 128, 4)
        ya = wq.gemm_offset(Xd, to_dev(c), to_dev(s), to_dev(m), N=N, K=K, group=128, bits=4)
        yu = wq.gemm_offset(Xd, to_dev(c), _offset_headers(s), _offset_headers(m), N=N, K=K, group=128, bits=4)
    else:
        bits = {"int4": 4, "int2": 2, "int3": 3}[fmt]
        c, s, z = oracle.quantize(W, 128, bits)
        ref = oracle.gemm(X, c, s, z, N, K, 128, bits)
        ya = wq.gemm(Xd, to_dev(c), to_dev(s), to_dev(z), N=N, K=K, group=128, bits=bits)
        yu = wq.gemm(Xd, to_dev(c), _offset_headers(s), _offset_headers(z), N=N, K=K, group=128, bits=bits)
    assert_close(ya, ref, f"{fmt} aligned")
    assert_close(yu, ref, f"{fmt} unaligned")
