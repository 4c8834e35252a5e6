"""GPU parity of wq_gemm (both kernel families) against the CPU oracle.

Inputs are quantized by the oracle (so the comparison isolates the product),
shapes span several tiles with ragged row, batch and chunk tails, and the
full-size workloads are checked on sampled output rows in the launch
configuration the benchmark times (automatic path selection).
"""

import numpy as np
import pytest

import oracle
import wq_inputs
from edge_groups import on_grid_matrix
from gpu_util import assert_close, device, note, to_dev, workload

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu


def packed(W, group, bits):
    c, s, z = oracle.quantize(W, group, bits)
    return (c, s, z), (to_dev(c), to_dev(s), to_dev(z))


def run(X, dev_packed, N, K, group, bits, path):
    c, s, z = dev_packed
    return wq.gemm(to_dev(X), c, s, z, N=N, K=K, group=group, bits=bits, path=path)


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (4, 256), (4, 1024), (8, 64), (8, 1024)])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 13])
def test_gemv_path(bits, group, B):
    device()
    rng = np.random.default_rng(B * 10 + bits)
    N, K = 203, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"gemv N={N} K={K} G={group} b={bits} B={B}")
    Y = run(X, dev, N, K, group, bits, "gemv")
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), "gemv")


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 256), (4, 1024), (8, 64), (8, 1024)])
@pytest.mark.parametrize("B", [1, 5, 16, 17, 32, 33, 64, 70, 130])
def test_mfma_path(bits, group, B):
    device()
    rng = np.random.default_rng(B * 10 + bits + 1)
    N, K = 203, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"mfma N={N} K={K} G={group} b={bits} B={B}")
    Y = run(X, dev, N, K, group, bits, "mfma")
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), "mfma")


@pytest.mark.parametrize("K,group,bits", [(896, 32, 4), (11008, 128, 4), (11008, 11008, 8),
                                          (4096, 4096, 8), (32, 32, 4), (16384, 128, 4)])
@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_gemv_row_lengths(K, group, bits, B):
    """Chunk counts from 1 to 1024 per row: every TG x CPT tiling, incl. LDS reductions."""
    device()
    rng = np.random.default_rng(K + B)
    N = 77
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"gemv row lengths N={N} K={K} G={group} b={bits} B={B}")
    Y = run(X, dev, N, K, group, bits, "gemv")
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), "gemv")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_on_grid_weights_match_library_matmul(path):
    """Weights on a quantization grid dequantize exactly, so Y_ref = X W^T."""
    device()
    W, _, _, _ = on_grid_matrix(130, 512, 128, 4, seed=11)
    rng = np.random.default_rng(12)
    X = rng.standard_normal((9, 512)).astype(np.float16)
    host, dev = packed(W, 128, 4)
    Y = run(X, dev, 130, 512, 128, 4, path)
    assert_close(Y, X.astype(np.float64) @ W.astype(np.float64).T, path)


@pytest.mark.parametrize("path,B", [("gemv", 4), ("mfma", 24)])
def test_row_permutation_is_bitwise(path, B):
    """Batch rows are independent: permuting X's rows permutes Y's rows exactly."""
    device()
    rng = np.random.default_rng(13)
    N, K = 150, 2048
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    _, dev = packed(W, 128, 4)
    perm = rng.permutation(B)
    Y = run(X, dev, N, K, 128, 4, path).cpu().numpy()
    Yp = run(X[perm], dev, N, K, 128, 4, path).cpu().numpy()
    assert np.array_equal(Yp.view(np.uint16), Y[perm].view(np.uint16))
    Y2 = run(X, dev, N, K, 128, 4, path).cpu().numpy()
    assert np.array_equal(Y2.view(np.uint16), Y.view(np.uint16))  # deterministic


def test_empty_and_degenerate_shapes():
    device()
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((5, 128)) * 0.02).astype(np.float16)
    host, dev = packed(W, 128, 4)
    Y = run(np.zeros((0, 128), np.float16), dev, 5, 128, 128, 4, "auto")
    assert tuple(Y.shape) == (0, 5)
    # Single group per row, single row.
    X = rng.standard_normal((3, 128)).astype(np.float16)
    c, s, z = host
    Y = wq.gemm(to_dev(X), to_dev(c[:1]), to_dev(s[:1]), to_dev(z[:1]), N=1, K=128, group=128,
                bits=4)
    assert_close(Y, oracle.gemm(X, c[:1], s[:1], z[:1], 1, 128, 128, 4), "N=1")


def test_large_activations_and_outliers():
    device()
    rng = np.random.default_rng(15)
    N, K = 96, 4096
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W.reshape(-1)[rng.choice(N * K, 400, replace=False)] = 0.5
    X = (rng.standard_normal((6, K)) * 200).astype(np.float16)
    host, dev = packed(W, 128, 4)
    for path in ("gemv", "mfma"):
        Y = run(X, dev, N, K, 128, 4, path)
        assert_close(Y, oracle.gemm(X, *host, N, K, 128, 4), path)


SAMPLE = 512


@pytest.mark.parametrize("name", list(wq_inputs.WORKLOADS))
def test_workload_full_size_sampled(name):
    """Full-size workloads at every batch of the workload, automatic path, sampled rows."""
    device()
    cfg = wq_inputs.WORKLOADS[name]
    N, K, G, bits = cfg["N"], cfg["K"], cfg["group"], cfg["bits"]
    W, X = workload(name)
    codes, scales, zeros = wq.quantize_pack(to_dev(W), G, bits)
    rows = np.unique(np.concatenate([np.random.default_rng(16).choice(N, SAMPLE, replace=False),
                                     [0, N - 1]]))
    # Rows are independent: the oracle quantizes and multiplies only the sample.
    hc, hs, hz = oracle.quantize(W[rows], G, bits)
    for B in cfg["batches"]:
        note(f"{name} B={B} auto path")
        Y = wq.gemm(to_dev(X[:B]), codes, scales, zeros, N=N, K=K, group=G, bits=bits)
        ref = oracle.gemm(X[:B], hc, hs, hz, len(rows), K, G, bits)
        assert_close(Y.cpu().numpy()[:, rows].astype(np.float64), ref, f"{name} B={B}")


@pytest.mark.parametrize("index", range(7))
def test_decode_set_layer0_b32(index):
    device()
    W, X = wq_inputs.decode_set_matrix(0, index)
    N, K = W.shape
    rows = np.random.default_rng(17).choice(N, 256, replace=False)
    for group, bits in ((128, 4), (K, 8)):
        note(f"decode-set #{index} G={group} b={bits} B=32")
        codes, scales, zeros = wq.quantize_pack(to_dev(W), group, bits)
        Y = wq.gemm(to_dev(X), codes, scales, zeros, N=N, K=K, group=group, bits=bits)
        ref = oracle.gemm(X, *oracle.quantize(W[rows], group, bits), len(rows), K, group, bits)
        assert_close(Y.cpu().numpy()[:, rows].astype(np.float64), ref, f"#{index} b={bits}")


def test_mlp70b_all_rows_every_metric_batch():
    """Every output of the 70B-class up-projection (28672 x 8192, group 128)
    at every batch size of the measured step, automatic path with and without
    a workspace, against the oracle's double-precision product."""
    device()
    name = "mlp70b_up_k8192_n28672_g128"
    cfg = wq_inputs.WORKLOADS[name]
    N, K, G = cfg["N"], cfg["K"], cfg["group"]
    W, X = workload(name)
    codes, scales, zeros = wq.quantize_pack(to_dev(W), G, 4)
    hc, hs, hz = oracle.quantize(W, G, 4)
    assert np.array_equal(codes.cpu().numpy(), hc)
    for B in (1, 2, 4, 8, 16, 32, 64):
        ref = oracle.gemm(X[:B], hc, hs, hz, N, K, G, 4)
        for use_ws in (True, False):
            note(f"{name} all rows B={B} workspace={use_ws}")
            Y = wq.gemm(to_dev(X[:B]), codes, scales, zeros, N=N, K=K, group=G, bits=4, use_workspace=use_ws)
            assert_close(Y, ref, f"{name} B={B} ws={use_ws}")
