"""wq_gemm_static, the product entry point that allocates nothing: its split
partials live in a static device array instead of a caller workspace.  Called
through the C ABI, it must give what wq_gemm_ex gives with a workspace (the
same plan and kernels, so bit for bit, and within the product tolerance of the
oracle), on two calls in a row whose second is smaller (the array keeps the
first call's contents), and must refuse a call whose plan needs more scratch
than the array holds, before any launch."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, device, note, to_dev

import bit_weight_only_wq_amd as wq
from bit_weight_only_wq_amd import _lib

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STATIC_BYTES = 16 << 20


def _ptrs(*ts):
    return [t.data_ptr() for t in ts]


def test_static_scratch_matches_workspace_entry_point():
    dev = device()
    lib = wq.load()
    stream = torch.cuda.current_stream().cuda_stream
    # (N, K, B, path): the X-resident kernel with two K-slices, then a smaller
    # product that splits K for parallelism (few rows), then the tiled kernel
    # with K splits.
    cases = [(300, 16384, 16, _lib.WQ_PATH_AUTO), (61, 8192, 5, _lib.WQ_PATH_AUTO),
             (200, 4096, 40, _lib.WQ_PATH_MFMA)]
    for N, K, B, path in cases:
        rng = np.random.default_rng(N * 7 + B)
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        X = rng.standard_normal((B, K)).astype(np.float16)
        host = oracle.quantize(W, 128, 4)
        c, s, z = (to_dev(a) for a in host)
        Xd = to_dev(X)
        need = wq.gemm_workspace_bytes(B, K, N, 128, 4, "auto" if path == 0 else "mfma")
        note(f"no-alloc N={N} K={K} B={B} path={path} scratch={need}")
        assert 0 < need <= STATIC_BYTES          # the scratch is really used
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        y_ws = torch.empty((B, N), dtype=torch.float16, device=dev)
        y_st = torch.full((B, N), float("nan"), dtype=torch.float16, device=dev)
        st = lib.wq_gemm_ex(*_ptrs(Xd, c, s, z, y_ws), B, K, N, 128, 4, path, ws.data_ptr(), need, stream)
        wq.check(st, "wq_gemm_ex")
        st = lib.wq_gemm_static(*_ptrs(Xd, c, s, z, y_st), B, K, N, 128, 4, path, stream)
        wq.check(st, "wq_gemm_static")
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_st.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (N, K, B)
        assert_close(b.astype(np.float64), oracle.gemm(X, *host, N, K, 128, 4), f"static N={N} B={B}")


def test_static_scratch_refuses_oversized_plans():
    """B = 64 on a 28672 x 16384 matrix (the tiled kernel, K split three ways)
    needs about 22 MB of partials: refused with WQ_ERR_UNSUPPORTED before
    anything is enqueued (real, if uninitialized, buffers, so nothing could go
    wrong even if it launched)."""
    dev = device()
    lib = wq.load()
    N, K, B = 28672, 16384, 64
    need = wq.gemm_workspace_bytes(B, K, N, 128, 4)
    note(f"no-alloc refusal need={need}")
    assert need > STATIC_BYTES
    X = torch.zeros((B, K), dtype=torch.float16, device=dev)
    c = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    s = torch.ones((N, K // 128), dtype=torch.float16, device=dev)
    z = torch.zeros((N, K // 128), dtype=torch.float16, device=dev)
    Y = torch.zeros((B, N), dtype=torch.float16, device=dev)
    st = lib.wq_gemm_static(*_ptrs(X, c, s, z, Y), B, K, N, 128, 4, 0, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.WQ_ERR_UNSUPPORTED
    assert b"static" in lib.wq_last_error()
    torch.cuda.synchronize()
    assert not Y.any()
