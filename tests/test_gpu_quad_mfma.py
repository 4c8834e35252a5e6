"""GPU parity of the 4x4x4 matrix-core kernels at B <= 4 on matrices of at
least 1024 rows against the CPU oracle: the quad-row kernel (wq_gemm_q4.hip)
takes groups of 32 (and group counts the quad-stream kernel cannot stage),
the quad-stream kernel (wq_gemm_qs.hip, its own tests) the rest.

What the geometry makes special: 4 rows walked in 512-k windows (K = 896 and
640 leave a partial last window, whose chunks past K read nothing), each
lane's 32-code chunk taking its own group header (groups of 32, 64, 128 and
256), batch rows past B as zero lanes of the A operand, N that is not a
multiple of 4 leaving a partial last quad, waves taking several quads in
turn.  Every output is compared.
"""

import numpy as np
import pytest

import oracle
import wq_inputs
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K, group)
    (4864, 896, 32),        # the 896 x 4864 GEMV workload's shape, group 32
    (1027, 640, 64),
    (2050, 4096, 128),
    (3001, 8192, 256),
    (1030, 11008, 128),     # 22 windows; 86 groups per row and a partial last quad
    (40000, 1024, 128),     # many quads per wave
]


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_quad_kernel_all_outputs(N, K, group, B):
    device()
    rng = np.random.default_rng(N + 5 * K + B)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    c, s, z = oracle.quantize(W, group, 4)
    ref = oracle.gemm(X, c, s, z, N, K, group, 4)
    note(f"quad-mfma N={N} K={K} G={group} B={B}")
    Y = wq.gemm(to_dev(X), to_dev(c), to_dev(s), to_dev(z), N=N, K=K, group=group, bits=4, path="mfma",
                use_workspace=False)
    assert_close(Y, ref, f"N={N} K={K} G={group} B={B}")


def test_groups_below_128_take_no_other_matrix_core_kernel():
    """Past B = 4 a group of 32 has no matrix-core kernel: the forced path is
    refused (the automatic path takes the GEMV)."""
    device()
    N, K = 1024, 896
    W = (np.random.default_rng(3).standard_normal((N, K)) * 0.02).astype(np.float16)
    c, s, z = (to_dev(a) for a in oracle.quantize(W, 32, 4))
    X = to_dev(np.ones((5, K), np.float16))
    with pytest.raises(wq.WQError):
        wq.gemm(X, c, s, z, N=N, K=K, group=32, bits=4, path="mfma")
    Y = wq.gemm(X, c, s, z, N=N, K=K, group=32, bits=4)
    assert Y.shape == (5, N)


def test_quad_kernel_on_the_first_workload_outliers():
    """The 7B-class up-projection (0.1 % outliers at +-0.5) at B = 1, 4, 8."""
    device()
    name = "mlp7b_up_k4096_n11008_g128"
    W, X = wq_inputs.workload_arrays(name)
    N, K = W.shape
    c, s, z = oracle.quantize(W, 128, 4)
    dev = [to_dev(a) for a in (c, s, z)]
    for B in (1, 4, 8):
        note(f"quad-mfma {name} B={B}")
        Y = wq.gemm(to_dev(X[:B]), *dev, N=N, K=K, group=128, bits=4, path="mfma")
        assert_close(Y, oracle.gemm(X[:B], c, s, z, N, K, 128, 4), f"{name} B={B}")
