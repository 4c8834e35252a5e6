"""Shared helpers of the GPU parity tests (HIP path vs CPU oracle)."""

import functools
import sys

import numpy as np
import pytest

import wq_inputs

torch = pytest.importorskip("torch")

# Tolerance on the product (fp32 accumulation, fp16 output), from the target
# definition: max|dY| <= 1e-2 * max|Y_ref| and ||dY|| / ||Y_ref|| <= 1e-3.
MAX_REL = 1e-2
L2_REL = 1e-3


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    """Print and flush what a GPU step is about to run (test, shape, path)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def assert_close(y_gpu, ref, what=""):
    """Compare a GPU fp16 output with the oracle's float64 result."""
    y = y_gpu.cpu().numpy().astype(np.float64) if hasattr(y_gpu, "cpu") else y_gpu
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), what
    scale = np.max(np.abs(ref))
    err = np.abs(y - ref)
    l2 = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    assert np.max(err) <= MAX_REL * scale, f"{what}: max|d|={np.max(err):.3e} vs {MAX_REL * scale:.3e}"
    assert l2 <= L2_REL, f"{what}: rel L2 {l2:.3e}"
    return l2


@functools.lru_cache(maxsize=2)
def workload(name):
    return wq_inputs.workload_arrays(name)
