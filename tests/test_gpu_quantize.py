"""GPU parity of wq_quantize_pack against the CPU oracle: codes, packed bytes,
scales and zero points must be bit-exact, on crafted corner-case groups, random
shapes, the full-size workloads and part of the 7B decode-step weight set.
Every code width 2..8 is covered (the little-endian bit stream per row), with
group sizes that take each kernel and each store width (whole 32-bit words,
single bytes)."""

import numpy as np
import pytest

import oracle
import wq_inputs
from edge_groups import crafted_groups, on_grid_matrix
from gpu_util import bits16, device, note, to_dev, workload

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu


def check_quantize(W, group, bits, what):
    device()
    note(f"quantize {what}: N={W.shape[0]} K={W.shape[1]} G={group} b={bits}")
    codes, scales, zeros = wq.quantize_pack(to_dev(W), group, bits)
    oc, os_, oz = oracle.quantize(W, group, bits)
    gc = codes.cpu().numpy()
    gs = bits16(scales.cpu().numpy())
    gz = bits16(zeros.cpu().numpy())
    assert np.array_equal(gs, bits16(os_)), f"{what}: scales differ ({np.sum(gs != bits16(os_))})"
    assert np.array_equal(gz, bits16(oz)), f"{what}: zeros differ ({np.sum(gz != bits16(oz))})"
    assert np.array_equal(gc, oc), f"{what}: codes differ ({np.sum(gc != oc)} bytes)"
    return codes, scales, zeros


ALL_BITS = [2, 3, 4, 5, 6, 7, 8]


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("group", [8, 16, 32, 64, 128, 256, 512, 96, 1024, 1536])
def test_crafted_groups(bits, group):
    W = crafted_groups(group, bits, seed=group)
    check_quantize(W, group, bits, "crafted")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("N,K,group", [(1, 8, 8), (3, 64, 32), (65, 512, 128), (7, 4096, 4096),
                                       (5, 11008, 11008), (33, 896, 32), (2, 1152, 384)])
def test_random_shapes(bits, N, K, group):
    rng = np.random.default_rng(N * 1000 + K)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 3.0])).astype(np.float16)
    check_quantize(W, group, bits, "random")


@pytest.mark.parametrize("bits", ALL_BITS)
def test_fixpoint_on_grid(bits):
    W, q, s, z = on_grid_matrix(16, 256, 32, bits)
    codes, scales, zeros = check_quantize(W, 32, bits, "on-grid")
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), s)
    assert np.array_equal(zeros.cpu().numpy().astype(np.float64), z.astype(np.float64))


@pytest.mark.parametrize("name", list(wq_inputs.WORKLOADS))
def test_workload_full_size(name):
    cfg = wq_inputs.WORKLOADS[name]
    W, _ = workload(name)
    check_quantize(W, cfg["group"], cfg["bits"], name)


@pytest.mark.parametrize("index", range(7))
def test_decode_set_layer0(index):
    W, _ = wq_inputs.decode_set_matrix(0, index)
    check_quantize(W, 128, 4, f"decode-set layer0 #{index} int4 g128")
    check_quantize(W, W.shape[1], 8, f"decode-set layer0 #{index} int8 per-channel")


def test_deterministic():
    W, _ = wq_inputs.decode_set_matrix(5, 4)
    d = to_dev(W)
    a = [t.cpu().numpy() for t in wq.quantize_pack(d, 128, 4)]
    b = [t.cpu().numpy() for t in wq.quantize_pack(d, 128, 4)]
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
