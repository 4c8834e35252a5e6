"""GPU parity of the one-batch-row GEMV kernel (B = 1) against the CPU oracle.

At B = 1, rows that fit one wave (up to 256 chunks of 16 bytes) and an even
number of groups per row take a kernel of their own: group headers read as
32-bit words (1, 2 or 4 per thread), a scalar row base when one row fills a
wave, and an all-zero X record for the chunks past a row's end.  The cases
below reach every thread-group width (16, 32, 64 threads per row), every
header-word count, ragged chunk counts, and the fallbacks to the general
kernel (odd group count, header arrays not 4-byte aligned).
"""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def packed(W, group, bits):
    c, s, z = oracle.quantize(W, group, bits)
    return (c, s, z), (to_dev(c), to_dev(s), to_dev(z))


# (K, group, bits): threads per row and header words per thread in comments.
CASES = [
    (8192, 128, 4),    # 64 threads, 1 word (the 70B-class up-projection's row)
    (8192, 64, 4),     # 64 threads, 2 words
    (8192, 32, 4),     # 64 threads, 4 words
    (6144, 128, 4),    # 192 chunks on 64 threads: 64 lanes read the zero record
    (6144, 64, 4),     # same, 2 words
    (4096, 128, 4),    # 32 threads (two rows per wave), 1 word
    (4096, 32, 4),     # 32 threads, 4 words
    (896, 32, 4),      # 16 threads, 28 chunks, 2 words
    (1024, 256, 4),    # 16 threads, 4 groups
    (4096, 64, 8),     # 8-bit, 64 threads, 1 word
    (4096, 16, 8),     # 8-bit, 64 threads, 4 words
    (2048, 128, 8),    # 8-bit, 32 threads
    (1040, 80, 8),     # 8-bit, 65 chunks on 32 threads, 13 groups: odd count, general kernel
    (4480, 128, 4),    # 35 groups: odd count, general kernel
]


@pytest.mark.parametrize("K,group,bits", CASES)
@pytest.mark.parametrize("N", [77, 1000])
def test_one_row_kernel(K, group, bits, N):
    device()
    rng = np.random.default_rng(K * 7 + group + bits + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((1, K)).astype(np.float16)
    host, dev = packed(W, group, bits)
    note(f"gemv B=1 N={N} K={K} G={group} b={bits}")
    Y = wq.gemm(to_dev(X), *dev, N=N, K=K, group=group, bits=bits, path="gemv")
    assert_close(Y, oracle.gemm(X, *host, N, K, group, bits), f"K={K} G={group} b={bits}")


def test_misaligned_headers_fall_back():
    """Header arrays that start 2 bytes past a 4-byte boundary take the
    general kernel and give the same result as aligned copies, bit for bit."""
    device()
    N, K, G = 300, 8192, 128
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    Xh = rng.standard_normal((1, K)).astype(np.float16)
    X = to_dev(Xh)
    host, (c, s, z) = packed(W, G, 4)
    ngrp = K // G
    sbuf = torch.zeros(N * ngrp + 1, dtype=torch.float16, device=s.device)
    zbuf = torch.zeros(N * ngrp + 1, dtype=torch.float16, device=s.device)
    sbuf[1:] = s.reshape(-1)
    zbuf[1:] = z.reshape(-1)
    s_odd = sbuf[1:].view(N, ngrp)
    z_odd = zbuf[1:].view(N, ngrp)
    assert s_odd.data_ptr() % 4 == 2
    note(f"gemv misaligned headers N={N} K={K}")
    y_al = wq.gemm(X, c, s, z, N=N, K=K, group=G, bits=4, path="gemv").cpu().numpy()
    y_mis = wq.gemm(X, c, s_odd, z_odd, N=N, K=K, group=G, bits=4, path="gemv").cpu().numpy()
    assert_close(y_mis.astype(np.float64), oracle.gemm(Xh, *host, N, K, G, 4), "misaligned")
    assert_close(y_al.astype(np.float64), y_mis.astype(np.float64), "aligned vs misaligned")
