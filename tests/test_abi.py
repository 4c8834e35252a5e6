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


def declared_functions():
    text = open(HEADER).read()
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


def test_version_and_status_strings():
    lib = wq.load()
    assert lib.wq_version() == 106
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
    return wq.load().wq_gemm_ex(X, C, S, Z, Y, B, K, N, group, bits, path, None)


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
    return wq.load().wq_quantize_pack_ex(W, N, K, group, bits, scheme, C, S, Z, None)


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
        assert lib.wq_gemm_grouped(arr, 3, None) == st
        assert b"item 2" in lib.wq_last_error()
    assert lib.wq_gemm_grouped(None, 2, None) == _lib.WQ_ERR_INVALID_ARG
    assert lib.wq_gemm_grouped(None, -1, None) == _lib.WQ_ERR_INVALID_ARG
    assert lib.wq_gemm_grouped(None, 0, None) == _lib.WQ_OK
    # No-op items (B == 0 or N == 0) are valid and enqueue nothing.
    arr = (_lib.GemmItem * 2)(_item(B=0), _item(N=0))
    assert lib.wq_gemm_grouped(arr, 2, None) == _lib.WQ_OK


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
    assert a(FAKE, None, FAKE, FAKE, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(max_blocks=0)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(heads=-1)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache()), 2, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache()), -1, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(0, FAKE, ctypes.byref(_cache()), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE + 8, FAKE, ctypes.byref(_cache()), 0, None) == _lib.WQ_ERR_MISALIGNED
    assert q(FAKE, FAKE, ctypes.byref(_cache(vcodes=0)), 0, None) == _lib.WQ_ERR_INVALID_ARG
    assert q(FAKE, FAKE, ctypes.byref(_cache(kres=FAKE + 2)), 0, None) == _lib.WQ_ERR_MISALIGNED
    assert a(FAKE, ctypes.byref(_cache()), 0, FAKE, None) == _lib.WQ_ERR_INVALID_ARG
    assert a(FAKE, ctypes.byref(_cache()), FAKE + 2, FAKE, None) == _lib.WQ_ERR_MISALIGNED
    assert a(FAKE + 1, ctypes.byref(_cache()), FAKE, FAKE, None) == _lib.WQ_ERR_MISALIGNED
    # No heads: nothing to do.
    assert q(0, 0, ctypes.byref(_cache(heads=0, kcodes=0)), 0, None) == _lib.WQ_OK
    assert a(0, ctypes.byref(_cache(heads=0)), 0, 0, None) == _lib.WQ_OK


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
