"""GPU parity of the streaming matrix-core kernel (B <= 16 on matrices of at
least 128 row tiles; wq_gemm_sk.hip) against the CPU oracle.

The kernel's own geometry makes these cases special: the 8 waves of a block
split K into 512-k positions (K = 640 and 11008 leave a partial last
position, K = 4096 gives every wave exactly one), a block owns up to 8 tiles
of 16 rows (ragged N leaves a partial last tile and a short last block), the
group headers are read either as 8-byte runs (group 128, aligned arrays) or
one entry per round (groups of 256 and 512, or arrays offset by one entry),
and batch rows past B are zero lanes of the matrix-core operand.  Every
output is compared, at batch sizes 1 to 16.
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = [  # (N, K, group)
    (2048 + 37, 4096, 128),
    (4100, 11008, 128),
    (2560, 640, 128),
    (3000, 8192, 256),
    (2048, 4096, 512),
    (33 * 256 * 8 + 5, 1024, 128),     # more tiles than 8 per compute unit: several blocks per CU
]


def _dev_headers(a, offset):
    """Device copy of a header array, optionally placed one entry past an
    8-byte boundary (the kernel then reads one entry per round)."""
    flat = torch.zeros(a.size + 4, dtype=torch.float16, device=device())
    flat[offset:offset + a.size] = to_dev(a.reshape(-1))
    return flat[offset:offset + a.size].view(a.shape)


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 13, 16])
def test_streaming_kernel_all_outputs(N, K, group, B):
    device()
    rng = np.random.default_rng(N + 3 * K + B)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((B, K)).astype(np.float16)
    c, s, z = oracle.quantize(W, group, 4)
    ref = oracle.gemm(X, c, s, z, N, K, group, 4)
    for offset in (0, 1):
        note(f"stream-mfma N={N} K={K} G={group} B={B} header offset={offset}")
        Y = wq.gemm(to_dev(X), to_dev(c), _dev_headers(s, offset), _dev_headers(z, offset),
                    N=N, K=K, group=group, bits=4, path="mfma", use_workspace=False)
        assert_close(Y, ref, f"N={N} K={K} G={group} B={B} off={offset}")


def test_streaming_kernel_is_deterministic_and_needs_no_workspace():
    device()
    N, K, B = 4100, 8192, 16
    assert wq.gemm_workspace_bytes(B, K, N, 128, 4, "mfma") == 0
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    Xd = to_dev(rng.standard_normal((B, K)).astype(np.float16))
    c, s, z = (to_dev(a) for a in oracle.quantize(W, 128, 4))
    note("stream-mfma repeat")
    y0 = wq.gemm(Xd, c, s, z, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
    y1 = wq.gemm(Xd, c, s, z, N=N, K=K, group=128, bits=4, path="mfma").cpu().numpy()
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))
