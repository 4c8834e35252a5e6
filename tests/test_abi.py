"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/wq.h declares, and rejects bad arguments synchronously (validation runs
before any HIP call, so none of these calls touches a device)."""

import os
import re

import pytest

from conftest import ROOT

wq = pytest.importorskip("bit_weight_only_wq_amd")
from bit_weight_only_wq_amd import _lib  # noqa: E402

HEADER = os.path.join(ROOT, "include", "wq.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = wq.load()
    names = declared_functions()
    assert "wq_quantize_pack" in names and "wq_gemm" in names
    for name in names:
        assert hasattr(lib, name), name
    # The Python binding declares a signature for each of them, and no others.
    assert sorted(_lib.SIGNATURES) == names


def test_probe_library_exports_its_header():
    """include/wq_probe.h is the read-stream probe's own library."""
    from bit_weight_only_wq_amd import probe
    lib = probe.load()
    names = declared_functions(os.path.join(ROOT, "include", "wq_probe.h"))
    assert names == ["wq_probe_read"]
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(probe.SIGNATURES) == names
    # Rejected before any launch: bad lane count, depth, order, shape, alignment.
    r = lambda **kw: lib.wq_probe_read(kw.get("buf", FAKE), kw.get("rows", 64), kw.get("row_bytes", 4096),
                                       kw.get("L", 16), kw.get("D", 8), kw.get("order", 0), 1, 2,
                                       kw.get("sink", FAKE), None)
    assert r(L=12) == 2
    assert r(D=3) == 2
    assert r(order=4) == 1
    assert r(rows=63) == 1                     # 4 rows per strip at L = 16
    assert r(row_bytes=4000) == 1
    assert r(buf=FAKE + 8) == 3
    assert r(buf=0) == 1


def test_version_and_status_strings():
    lib = wq.load()
    assert lib.wq_version() == 200
    for st in range(5):
        assert lib.wq_status_string(st)
    assert lib.wq_status_string(99) == b"unknown status"


def test_size_helpers():
    lib = wq.load()
    assert lib.wq_codes_bytes(11008, 4096, 4) == 11008 * 4096 // 2
    assert lib.wq_codes_bytes(4096, 11008, 8) == 4096 * 11008
    assert lib.wq_codes_bytes(-1, 8, 4) == 0
    assert lib.wq_num_groups(28672, 8192, 128) == 28672 * 64
    assert lib.wq_num_groups(4, 100, 128) == -1


FAKE = 0x100000  # 16-byte aligned, never dereferenced (validation fails first)


def _gemm(B=4, K=256, N=64, group=128, bits=4, path=0, X=FAKE, C=FAKE, S=FAKE, Z=FAKE, Y=FAKE):
    return wq.load().wq_gemm_ex(X, C, S, Z, Y, B, K, N, group, bits, path, None, 0, None)


def _quant(N=64, K=256, group=128, bits=4, W=FAKE, C=FAKE, S=FAKE, Z=FAKE):
    return wq.load().wq_quantize_pack(W, N, K, group, bits, C, S, Z, None)


def test_gemm_validation_errors():
    assert _gemm(K=250) == _lib.WQ_ERR_INVALID_ARG          # K % group
    assert _gemm(B=-1) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(K=0) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(group=0) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(bits=5) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=1) == _lib.WQ_ERR_UNSUPPORTED
    # 2/3 bits: 32-code chunks in one group, rows of whole 16-byte loads,
    # GEMV path only (all rejected before any launch).
    assert _gemm(bits=3, K=192, group=64) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=2, K=256, group=16) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=2, K=32, group=32) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=2, path=_lib.WQ_PATH_MFMA) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=3, K=65536, group=128) == _lib.WQ_ERR_UNSUPPORTED
    assert _gemm(bits=3, C=FAKE + 8) == _lib.WQ_ERR_MISALIGNED
    assert _gemm(bits=9) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(path=7) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(group=16, K=256) == _lib.WQ_ERR_UNSUPPORTED  # chunk spans groups
    assert _gemm(X=0) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(Y=0) == _lib.WQ_ERR_INVALID_ARG
    assert _gemm(X=FAKE + 8) == _lib.WQ_ERR_MISALIGNED
    assert _gemm(C=FAKE + 4) == _lib.WQ_ERR_MISALIGNED
    assert _gemm(Y=FAKE + 1) == _lib.WQ_ERR_MISALIGNED
    # The MFMA path needs group % 128 at 4 bits.
    assert _gemm(group=32, path=_lib.WQ_PATH_MFMA) == _lib.WQ_ERR_UNSUPPORTED
    assert wq.load().wq_last_error()


def test_empty_calls_are_no_ops():
    assert _gemm(B=0, X=0, Y=0) == _lib.WQ_OK
    assert _gemm(N=0, C=0, S=0, Z=0, Y=0) == _lib.WQ_OK
    assert _quant(N=0, W=0, C=0, S=0, Z=0) == _lib.WQ_OK


def test_quantize_validation_errors():
    assert _quant(K=250) == _lib.WQ_ERR_INVALID_ARG
    assert _quant(bits=0) == _lib.WQ_ERR_INVALID_ARG
    assert _quant(bits=1) == _lib.WQ_ERR_UNSUPPORTED
    assert _quant(group=4, K=256) == _lib.WQ_ERR_UNSUPPORTED
    assert _quant(W=0) == _lib.WQ_ERR_INVALID_ARG
    assert _quant(W=FAKE + 2) == _lib.WQ_ERR_MISALIGNED
    assert _quant(bits=8, C=FAKE + 4) == _lib.WQ_ERR_MISALIGNED
    assert _quant(bits=4, C=FAKE + 8) == _lib.WQ_ERR_MISALIGNED


def _quant_ex(scheme, N=64, K=256, group=128, bits=4, W=FAKE, C=FAKE, S=FAKE, Z=FAKE):
    return wq.load().wq_quantize_pack_ex(W, N, K, group, bits, scheme, C, S, Z, None, 0, None)


def test_quantize_ex_validation_errors():
    for scheme in (_lib.WQ_SCHEME_SYM, _lib.WQ_SCHEME_SYM_TENSOR):
        assert _quant_ex(scheme, N=0, W=0, C=0, S=0, Z=0) == _lib.WQ_OK
        assert _quant_ex(scheme, K=250) == _lib.WQ_ERR_INVALID_ARG
        assert _quant_ex(scheme, bits=1) == _lib.WQ_ERR_UNSUPPORTED
        assert _quant_ex(scheme, W=0) == _lib.WQ_ERR_INVALID_ARG
        assert _quant_ex(scheme, W=FAKE + 2) == _lib.WQ_ERR_MISALIGNED
    assert _quant_ex(5) == _lib.WQ_ERR_INVALID_ARG
    assert _quant_ex(-1) == _lib.WQ_ERR_INVALID_ARG
    assert b"scheme" in wq.load().wq_last_error()


def test_binding_raises_on_error():
    with pytest.raises(wq.WQError):
        _lib.check(_gemm(K=250), "wq_gemm")


def _item(B=4, K=256, N=64, group=128, bits=4, X=FAKE, C=FAKE, S=FAKE, Z=FAKE, Y=FAKE):
    return _lib.GemmItem(X, C, S, Z, Y, B, K, N, group, bits)


def test_grouped_validates_every_item_first():
    """An invalid item anywhere makes the whole call fail before any launch;
    the error names the item."""
    lib = wq.load()
    for bad, st in [(dict(K=200), _lib.WQ_ERR_INVALID_ARG), (dict(bits=5), _lib.WQ_ERR_UNSUPPORTED),
                    (dict(X=FAKE + 2), _lib.WQ_ERR_MISALIGNED), (dict(Y=0), _lib.WQ_ERR_INVALID_ARG)]:
        arr = (_lib.GemmItem * 3)(_item(), _item(B=32), _item(**bad))
        assert lib.wq_gemm_grouped(arr, 3, None, 0, None) == st
        assert b"item 2" in lib.wq_last_error()
    assert lib.wq_gemm_grouped(None, 2, None, 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert lib.wq_gemm_grouped(None, -1, None, 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert lib.wq_gemm_grouped(None, 0, None, 0, None) == _lib.WQ_OK
    # No-op items (B == 0 or N == 0) are valid and enqueue nothing.
    arr = (_lib.GemmItem * 2)(_item(B=0), _item(N=0))
    assert lib.wq_gemm_grouped(arr, 2, None, 0, None) == _lib.WQ_OK


def _cache(heads=4, max_blocks=2, **kw):
    f = dict(kcodes=FAKE, kscales=FAKE, kzeros=FAKE, vcodes=FAKE, vscales=FAKE, vzeros=FAKE,
             kres=FAKE, vres=FAKE)
    f.update(kw)
    return _lib.KvCache(f["kcodes"], f["kscales"], f["kzeros"], f["vcodes"], f["vscales"],
                        f["vzeros"], f["kres"], f["vres"], heads, max_blocks)


def test_kv_validation_errors():
    import ctypes
    lib = wq.load()
    q = lib.wq_kv_quantize_block
    a = lib.wq_kv_attention
    assert q(FAKE, FAKE, None, 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert a(FAKE, None, FAKE, FAKE, None, 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(max_blocks=0)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(heads=-1)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache()), 2, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache()), -1, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(0, FAKE, ctypes.byref(_cache()), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE + 8, FAKE, ctypes.byref(_cache()), 0, None) == _lib.WQ_ERR_MISALIGNED
    assert q(FAKE, FAKE, ctypes.byref(_cache(vcodes=0)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(kres=FAKE + 2)), 0, None) == _lib.WQ_ERR_MISALIGNED
    assert a(FAKE, ctypes.byref(_cache()), 0, FAKE, None, 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert a(FAKE, ctypes.byref(_cache()), FAKE + 2, FAKE, None, 0, None) == _lib.WQ_ERR_MISALIGNED
    assert a(FAKE + 1, ctypes.byref(_cache()), FAKE, FAKE, None, 0, None) == _lib.WQ_ERR_MISALIGNED
    # No heads: nothing to do.
    assert q(0, 0, ctypes.byref(_cache(heads=0, kcodes=0)), 0, None) == _lib.WQ_OK
    assert a(0, ctypes.byref(_cache(heads=0)), 0, 0, None, 0, None) == _lib.WQ_OK


def test_nf4_validation_errors():
    lib = wq.load()
    g = lambda **kw: lib.wq_gemm_nf4(kw.get("X", FAKE), kw.get("C", FAKE), kw.get("S", FAKE),
                                     kw.get("Y", FAKE), kw.get("B", 2), kw.get("K", 256),
                                     kw.get("N", 64), kw.get("group", 64), None)
    assert g(K=250) == _lib.WQ_ERR_INVALID_ARG
    assert g(group=16, K=256) == _lib.WQ_ERR_UNSUPPORTED
    assert g(K=32768, group=64) == _lib.WQ_ERR_UNSUPPORTED
    assert g(X=0) == _lib.WQ_ERR_INVALID_ARG
    assert g(X=FAKE + 8) == _lib.WQ_ERR_MISALIGNED
    assert g(B=0, X=0, Y=0) == _lib.WQ_OK
    assert _quant_ex(_lib.WQ_SCHEME_NF4, bits=3) == _lib.WQ_ERR_UNSUPPORTED
    assert _quant_ex(_lib.WQ_SCHEME_OFFSET + 1) == _lib.WQ_ERR_INVALID_ARG


def test_offset_gemm_validation_errors():
    lib = wq.load()
    g = lambda **kw: lib.wq_gemm_offset(kw.get("X", FAKE), FAKE, FAKE, kw.get("M", FAKE), kw.get("Y", FAKE),
                                        kw.get("B", 2), kw.get("K", 256), 64, kw.get("group", 64),
                                        kw.get("bits", 4), None)
    assert g(bits=5) == _lib.WQ_ERR_UNSUPPORTED
    assert g(bits=0) == _lib.WQ_ERR_INVALID_ARG
    assert g(group=16) == _lib.WQ_ERR_UNSUPPORTED
    assert g(bits=3, K=192, group=64) == _lib.WQ_ERR_UNSUPPORTED
    assert g(K=250) == _lib.WQ_ERR_INVALID_ARG
    assert g(M=0) == _lib.WQ_ERR_INVALID_ARG
    assert g(M=FAKE + 1) == _lib.WQ_ERR_MISALIGNED
    assert g(B=0, X=0, Y=0) == _lib.WQ_OK


def _deq(scheme=0, N=64, K=256, group=128, bits=4, C=FAKE, S=FAKE, Z=FAKE, W=FAKE):
    return wq.load().wq_dequantize(C, S, Z, N, K, group, bits, scheme, W, None)


def test_dequantize_validation_errors():
    """Every call here fails validation (or is the N = 0 no-op), so the fake
    pointers are never used."""
    for scheme in range(5):
        assert _deq(scheme, N=0, C=0, S=0, Z=0, W=0) == _lib.WQ_OK
        assert _deq(scheme, K=250) == _lib.WQ_ERR_INVALID_ARG
        assert _deq(scheme, N=-1) == _lib.WQ_ERR_INVALID_ARG
        assert _deq(scheme, bits=1) == _lib.WQ_ERR_UNSUPPORTED
        assert _deq(scheme, bits=9) == _lib.WQ_ERR_UNSUPPORTED
        assert _deq(scheme, group=4, K=256) == _lib.WQ_ERR_UNSUPPORTED
        assert _deq(scheme, C=0) == _lib.WQ_ERR_INVALID_ARG
        assert _deq(scheme, W=0) == _lib.WQ_ERR_INVALID_ARG
        assert _deq(scheme, W=FAKE + 4) == _lib.WQ_ERR_MISALIGNED
        assert _deq(scheme, S=FAKE + 1) == _lib.WQ_ERR_MISALIGNED
    assert _deq(5) == _lib.WQ_ERR_INVALID_ARG
    assert _deq(-1) == _lib.WQ_ERR_INVALID_ARG
    assert _deq(_lib.WQ_SCHEME_NF4, bits=3) == _lib.WQ_ERR_UNSUPPORTED
    assert b"wq_dequantize" in wq.load().wq_last_error()


# ---- caller-owned workspace -------------------------------------------------


def _gemm_ws_size(B, K=8192, N=28672, group=128, bits=4, path=0):
    import ctypes
    n = ctypes.c_size_t(123)
    st = wq.load().wq_gemm_workspace_size(B, K, N, group, bits, path, ctypes.byref(n))
    return st, n.value


def test_gemm_workspace_size_queries():
    """The size query validates the shape like the call and reports the bytes
    of the split partials the preferred plan writes (0 when it has none)."""
    st, n = _gemm_ws_size(1)
    assert st == _lib.WQ_OK and n == 0                   # GEMV: no scratch
    st, n = _gemm_ws_size(16)
    assert st == _lib.WQ_OK and n == 0                   # tall matrix at B = 16: streaming kernel, no scratch
    st, n = _gemm_ws_size(16, K=16384, N=300)
    assert st == _lib.WQ_OK and n > 0 and n % (16 * 300 * 4) == 0     # few rows: K-slices in partials
    st, n = _gemm_ws_size(64)
    assert st == _lib.WQ_OK and n == 0                   # tall matrix at B = 64: K-split waves, no scratch
    st, n = _gemm_ws_size(64, K=16384)
    assert st == _lib.WQ_OK and n > 0 and n % (64 * 28672 * 4) == 0   # tiled kernel's K splits
    st, n = _gemm_ws_size(0)
    assert st == _lib.WQ_OK and n == 0                   # no-op
    st, n = _gemm_ws_size(16, K=250)
    assert st == _lib.WQ_ERR_INVALID_ARG and n == 0
    st, n = _gemm_ws_size(2, bits=5)
    assert st == _lib.WQ_ERR_UNSUPPORTED and n == 0
    assert wq.load().wq_gemm_workspace_size(1, 256, 64, 128, 4, 0, None) == _lib.WQ_ERR_INVALID_ARG


def test_gemm_workspace_rejected_before_launch():
    """An undersized, misaligned, or null-with-a-size workspace is refused
    before anything is enqueued (the fake pointers are never used)."""
    lib = wq.load()
    st, need = _gemm_ws_size(64, K=16384)
    assert need > 0
    call = lambda ws, n: lib.wq_gemm_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 16384, 28672, 128, 4, 0, ws, n, None)
    assert call(FAKE, need - 1) == _lib.WQ_ERR_INVALID_ARG
    assert b"needs" in lib.wq_last_error()
    assert call(FAKE, 0) == _lib.WQ_ERR_INVALID_ARG
    assert call(None, 64) == _lib.WQ_ERR_INVALID_ARG
    assert call(FAKE + 8, need) == _lib.WQ_ERR_MISALIGNED
    # A no-op call accepts no workspace and rejects a bad one.
    noop = lambda ws, n: lib.wq_gemm_ex(0, FAKE, FAKE, FAKE, 0, 0, 8192, 28672, 128, 4, 0, ws, n, None)
    assert noop(None, 0) == _lib.WQ_OK
    assert noop(None, 8) == _lib.WQ_ERR_INVALID_ARG


def test_grouped_workspace_size_and_rejection():
    import ctypes
    lib = wq.load()
    arr = (_lib.GemmItem * 2)(_item(B=16, K=16384, N=300), _item(B=1, K=8192, N=28672))
    n = ctypes.c_size_t(0)
    assert lib.wq_gemm_grouped_workspace_size(arr, 2, ctypes.byref(n)) == _lib.WQ_OK
    assert n.value > 0
    assert lib.wq_gemm_grouped(arr, 2, FAKE, n.value - 16, None) == _lib.WQ_ERR_INVALID_ARG
    bad = (_lib.GemmItem * 1)(_item(K=200))
    assert lib.wq_gemm_grouped_workspace_size(bad, 1, ctypes.byref(n)) == _lib.WQ_ERR_INVALID_ARG
    assert b"item 0" in lib.wq_last_error()


def test_kv_and_quantize_workspace():
    import ctypes
    lib = wq.load()
    n = ctypes.c_size_t(0)
    # Few heads, long context: the attention splits the context.
    assert lib.wq_kv_workspace_size(ctypes.byref(_cache(heads=32, max_blocks=256)), ctypes.byref(n)) == _lib.WQ_OK
    assert n.value > 0 and n.value % (32 * (128 + 4) * 4) == 0
    need = n.value
    a = lib.wq_kv_attention
    assert a(FAKE, ctypes.byref(_cache(heads=32, max_blocks=256)), FAKE, FAKE, FAKE, need - 4, None) == \
        _lib.WQ_ERR_INVALID_ARG
    assert lib.wq_kv_workspace_size(ctypes.byref(_cache(heads=0)), ctypes.byref(n)) == _lib.WQ_OK and n.value == 0
    # The per-tensor symmetric quantizer needs scratch for its maximum.
    for scheme, want in ((_lib.WQ_SCHEME_ASYM, 0), (_lib.WQ_SCHEME_SYM_TENSOR, 4100)):
        assert lib.wq_quantize_workspace_size(64, 256, 128, 4, scheme, ctypes.byref(n)) == _lib.WQ_OK
        assert n.value == want
    q = lambda ws, nb: lib.wq_quantize_pack_ex(FAKE, 64, 256, 128, 4, _lib.WQ_SCHEME_SYM_TENSOR, FAKE, FAKE,
                                               FAKE, ws, nb, None)
    assert q(None, 0) == _lib.WQ_ERR_INVALID_ARG
    assert b"workspace" in lib.wq_last_error()
    assert q(FAKE, 4099) == _lib.WQ_ERR_INVALID_ARG


def test_library_sources_allocate_nothing():
    """The HIP sources call no device or host allocator: every buffer is the
    caller's."""
    src = os.path.join(ROOT, "bit_weight_only_wq_amd", "csrc")
    pat = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipMallocManaged|hipExtMallocWithFlags)\s*\(")
    for dirpath, _, files in os.walk(src):
        for f in files:
            if f.endswith((".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f
