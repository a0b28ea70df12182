"""Host-side checks of libfp4idx.so (no GPU needed).

The library loads, exports every symbol include/fp4idx.h declares, and rejects bad
arguments on the host before anything is enqueued (every call here returns before the
first HIP runtime call).
"""
import ctypes
import os
import re

import pytest

from sparse_attention_fp4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    with open(os.path.join(ROOT, "include", "fp4idx.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fp4idx_\w+)\s*\(", src, re.M)))


def test_header_declares_exactly_the_binding_exports():
    assert header_symbols() == sorted(_lib.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    L = _lib.lib()
    for name in header_symbols():
        assert hasattr(L, name), name
    assert L.fp4idx_version() == 100
    for code in range(6):
        assert L.fp4idx_strerror(code)


def test_topk_wait_limit_setter():
    """The bound on the one-kernel top-k's in-memory waits: each call returns the previous
    bound, a negative value only reads it (no GPU call is made)."""
    L = _lib.lib()
    prev = L.fp4idx_set_topk_wait_limit(-1)
    assert prev == 65536
    try:
        assert L.fp4idx_set_topk_wait_limit(0) == prev
        assert L.fp4idx_set_topk_wait_limit(123) == 0
        assert L.fp4idx_set_topk_wait_limit(-5) == 123
        assert L.fp4idx_set_topk_wait_limit(-1) == 123
    finally:
        L.fp4idx_set_topk_wait_limit(prev)
    assert L.fp4idx_set_topk_wait_limit(-1) == prev


def _logits(**kw):
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p).value
    p16 = (p + 255) & ~255
    a = dict(fmt=0, q=p16, qrs=32 * 64, qs=p16, qsrs=32 * 4, w=p16, wrs=32, k=p16,
             kps=64 * 64, ks=p16, ksps=64 * 4, bt=p16, btrs=4, cu=p16, lens=p16, T=4, B=1, H=32,
             Hkv=1, page=64, P=4, W=4, out_cols=256, out=p16, ors=256, stream=None)
    a.update(kw)
    return L.fp4idx_logits_paged(a["fmt"], a["q"], a["qrs"], a["qs"], a["qsrs"], a["w"], a["wrs"],
                                 a["k"], a["kps"], a["ks"], a["ksps"], a["bt"], a["btrs"], a["cu"],
                                 a["lens"], a["T"], a["B"], a["H"], a["Hkv"], a["page"], a["P"],
                                 a["W"], a["out_cols"], a["out"], a["ors"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=2), 1), (dict(H=6, Hkv=4), 1), (dict(page=32), 2), (dict(H=256, qrs=256 * 64,
     qsrs=256 * 4, wrs=256), 2), (dict(q=None), 1), (dict(B=0), 1), (dict(qrs=100), 1),
    (dict(qrs=32 * 64 + 8), 3), (dict(out_cols=300), 1), (dict(kps=100), 1),
    (dict(ors=(1 << 27) + 4), 2),
])
def test_logits_argument_errors(kw, code):
    assert _logits(**kw) == code


def test_logits_empty_work_is_ok_without_launch():
    assert _logits(T=0) == 0
    assert _logits(out_cols=0, ors=0) == 0


def _blocks(**kw):
    L = _lib.lib()
    a = dict(fmt=1, q=256, qs=256, k=256, ks=256, cuq=256, cuk=256, cup=256, kvi=256, qo=None,
             B=1, Tq=4, Hq=8, Hkv=2, P=4, msq=4, msk=300, causal=1, out=256)
    a.update(kw)
    return L.fp4idx_block_scores(a["fmt"], a["q"], a["qs"], a["k"], a["ks"], a["cuq"], a["cuk"],
                                 a["cup"], a["kvi"], a["qo"], a["B"], a["Tq"], a["Hq"], a["Hkv"],
                                 a["P"], a["msq"], a["msk"], a["causal"], a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(msq=0), 1), (dict(Hq=8, Hkv=3), 1), (dict(qo=256, causal=0), 1), (dict(fmt=-1), 1),
    (dict(q=None), 1), (dict(q=264), 3),
])
def test_block_score_argument_errors(kw, code):
    assert _blocks(**kw) == code


def test_topk_argument_errors_and_workspace():
    L = _lib.lib()
    assert L.fp4idx_topk(256, 10, 2, 10, None, 0, 256, None, None, 0, None) == 1      # k < 1
    assert L.fp4idx_topk(256, 10, 2, 10, None, 9000, 256, None, None, 0, None) == 2   # k too big
    assert L.fp4idx_topk(256, 1 << 20, 1, 1 << 20, None, 8, 256, None, None, 0, None) == 2  # cols
    assert L.fp4idx_topk(256, 5, 2, 10, None, 4, 256, None, None, 0, None) == 1       # stride
    assert L.fp4idx_topk_workspace_bytes(4, 8192, 2048) == 0                         # one workgroup a row
    assert L.fp4idx_topk_workspace_bytes(65, 32768, 2048) == 0
    assert L.fp4idx_topk_workspace_bytes(64, 8193, 2048) > 0                         # chunked
    assert L.fp4idx_topk_workspace_bytes(600, 32769, 2048) > 0
    need = L.fp4idx_topk_workspace_bytes(4, 100_000, 2048)
    assert need > 0
    assert L.fp4idx_topk(256, 100_000, 4, 100_000, None, 2048, 256, None, None, 0, None) == 5
    assert L.fp4idx_topk(256, 100_000, 4, 100_000, None, 2048, 256, None, 512 + 8, need,
                         None) == 5                                                  # misaligned


def test_quantize_store_argument_errors():
    L = _lib.lib()
    f = L.fp4idx_quantize_store_k
    assert f(256, 128, 256, -1, 256, 4096, 256, 256, 64, 4, None) == 1       # N < 0
    assert f(256, 128, 256, 4, 256, 4096, 256, 256, 32, 4, None) == 2        # page size
    assert f(256, 128, 256, 0, 256, 4096, 256, 256, 64, 4, None) == 0        # nothing to do
    assert f(None, 128, 256, 4, 256, 4096, 256, 256, 64, 4, None) == 1       # null keys
    assert f(256, 100, 256, 4, 256, 4096, 256, 256, 64, 4, None) == 1        # short rows
    assert f(258, 128, 256, 4, 256, 4096, 256, 256, 64, 4, None) == 3        # misaligned
    assert f(256, 129, 256, 4, 256, 4096, 256, 256, 64, 4, None) == 3        # odd stride


def test_block_topk_argument_errors():
    L = _lib.lib()
    f = L.fp4idx_block_topk
    assert f(256, 0, 4, 8, 2, 256, None, None) == 1        # Hq < 1
    assert f(256, 2, -1, 8, 2, 256, None, None) == 1       # Ktiles < 0
    assert f(256, 2, 4, 8, 0, 256, None, None) == 1        # k < 1
    assert f(256, 2, 4, 8, 65, 256, None, None) == 2       # k > 64
    assert f(256, 2, 4, 0, 2, 256, None, None) == 0        # no queries: nothing to do
    assert f(None, 2, 4, 8, 2, 256, None, None) == 1       # missing scores
    assert f(256, 2, 4, 8, 2, None, None, None) == 1       # missing output


def _qsa_slots(**kw):
    L = _lib.lib()
    a = dict(ind=256, irs=9, rows=4, topk=8, bt=256, btrs=4, nreq=2, width=4, t2r=256, nb=16,
             page=64, slots=256, srs=8, cols=8)
    a.update(kw)
    return L.fp4idx_qsa_slots(a["ind"], a["irs"], a["rows"], a["topk"], a["bt"], a["btrs"],
                              a["nreq"], a["width"], a["t2r"], a["nb"], a["page"], a["slots"],
                              a["srs"], a["cols"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 1), (dict(topk=0), 1), (dict(cols=7), 1), (dict(page=0), 1),
    (dict(nreq=0), 1), (dict(width=0), 1), (dict(nb=0), 1), (dict(irs=7), 1),
    (dict(btrs=3), 1), (dict(srs=7), 1), (dict(ind=None), 1), (dict(slots=None), 1),
    (dict(nb=1 << 25, page=64), 1),          # 2^25 pages << 6 bits does not fit in int32
    (dict(rows=0, ind=None), 0),             # nothing to do
])
def test_qsa_slots_argument_errors(kw, code):
    assert _qsa_slots(**kw) == code


def _qsa_decode(**kw):
    L = _lib.lib()
    a = dict(q=256, qrs=32 * 128, qhs=128, k=256, v=256 + 128, bs=4 * 64 * 256, ts=256,
             khs=64 * 256, vhs=64 * 256, nb=16, page=64, slots=256, srs=8, ind=256, irs=9,
             topk=8, rows=4, Hq=32, Hkv=4, D=128, ss=0.1, os=1.0, gate=256, grs=32 * 128,
             ghs=128, out=256, ors=32 * 128, ohs=128)
    a.update(kw)
    return L.fp4idx_qsa_decode(a["q"], a["qrs"], a["qhs"], a["k"], a["v"], a["bs"], a["ts"],
                               a["khs"], a["vhs"], a["nb"], a["page"], a["slots"], a["srs"],
                               a["ind"], a["irs"], a["topk"], a["rows"], a["Hq"], a["Hkv"],
                               a["D"], a["ss"], a["os"], a["gate"], a["grs"], a["ghs"],
                               a["out"], a["ors"], a["ohs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 1), (dict(topk=0), 1), (dict(Hkv=0), 1), (dict(Hq=30), 1),
    (dict(Hq=2), 1), (dict(page=0), 1), (dict(nb=0), 1), (dict(irs=8), 1),
    (dict(q=None), 1), (dict(gate=None), 1), (dict(out=None), 1), (dict(slots=None), 1),
    (dict(nb=1 << 25), 1),
    (dict(D=64), 2), (dict(Hq=68, Hkv=4), 2), (dict(bs=1 << 32), 2), (dict(ts=1 << 32), 2),
    (dict(q=264), 3), (dict(k=264), 3), (dict(v=256 + 136), 3), (dict(out=258), 3),
    (dict(qhs=132), 3), (dict(ors=32 * 128 + 4), 3), (dict(ts=264), 3), (dict(vhs=8), 3),
    (dict(rows=0, q=None), 0),               # nothing to do
])
def test_qsa_decode_argument_errors(kw, code):
    assert _qsa_decode(**kw) == code


def _fused(ws_bytes=None, ws_off=0, **kw):
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p).value
    p16 = (p + 255) & ~255
    a = dict(fmt=0, q=p16, qrs=32 * 64, qs=p16, qsrs=32 * 4, w=p16, wrs=32, k=p16,
             kps=64 * 64, ks=p16, ksps=64 * 4, bt=p16, btrs=4, cu=p16, lens=p16, T=4, B=1, H=32,
             Hkv=1, page=64, P=4, W=4, out_cols=256, kk=16, idx=p16, vals=None)
    a.update(kw)
    need = L.fp4idx_logits_topk_workspace_bytes(a["fmt"], a["T"], a["B"], a["H"], a["Hkv"],
                                                a["page"], a["W"], a["out_cols"], a["kk"])
    return L.fp4idx_logits_topk_paged(
        a["fmt"], a["q"], a["qrs"], a["qs"], a["qsrs"], a["w"], a["wrs"], a["k"], a["kps"],
        a["ks"], a["ksps"], a["bt"], a["btrs"], a["cu"], a["lens"], a["T"], a["B"], a["H"],
        a["Hkv"], a["page"], a["P"], a["W"], a["out_cols"], a["kk"], a["idx"], a["vals"],
        p16 + ws_off if ws_bytes != 0 else None, need if ws_bytes is None else ws_bytes, None)


def test_logits_topk_workspace_size():
    L = _lib.lib()
    f = L.fp4idx_logits_topk_workspace_bytes
    small = f(0, 4, 1, 32, 1, 64, 32, 2048, 256)
    big = f(0, 4, 1, 32, 1, 64, 64, 4096, 256)
    assert 0 < small < big
    # fewer than 512 rows: the logits themselves (4 bytes per column and row) and the
    # top-k's histograms; 512 rows or more: the kept-score buffer (8 bytes each)
    assert big >= 4 * 4096 * 4
    assert f(0, 600, 2, 32, 1, 64, 64, 4096, 256) >= 600 * 4096 * 8
    assert f(0, 4, 1, 30, 4, 64, 32, 2048, 256) == 0       # H % Hkv != 0
    assert f(0, 4, 1, 32, 1, 32, 32, 2048, 256) == 0       # page size
    assert f(0, 0, 1, 32, 1, 64, 32, 2048, 256) == 0       # no rows


@pytest.mark.parametrize("kw,code", [
    (dict(kk=0), 1), (dict(kk=2049), 2), (dict(out_cols=(1 << 24) + 64), 2), (dict(fmt=3), 1),
    (dict(H=6, Hkv=4), 1), (dict(page=32), 2), (dict(idx=None), 1), (dict(q=None), 1),
    (dict(qrs=32 * 64 + 8), 3), (dict(ws_bytes=0), 5), (dict(ws_bytes=64), 5),
    (dict(ws_off=16), 5), (dict(T=0), 0),
])
def test_logits_topk_argument_errors(kw, code):
    assert _fused(**kw) == code


def _noalloc(**kw):
    L = _lib.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p).value
    p16 = (p + 255) & ~255
    a = dict(fmt=0, q=p16, qrs=32 * 64, qs=p16, qsrs=32 * 4, w=p16, wrs=32, k=p16,
             kps=64 * 64, ks=p16, ksps=64 * 4, bt=p16, btrs=4, cu=p16, lens=p16, T=4, B=1, H=32,
             Hkv=1, page=64, P=4, W=4, out_cols=256, kk=16, idx=p16, vals=None)
    a.update(kw)
    return L.fp4idx_logits_topk_paged_noalloc(
        a["fmt"], a["q"], a["qrs"], a["qs"], a["qsrs"], a["w"], a["wrs"], a["k"], a["kps"],
        a["ks"], a["ksps"], a["bt"], a["btrs"], a["cu"], a["lens"], a["T"], a["B"], a["H"],
        a["Hkv"], a["page"], a["P"], a["W"], a["out_cols"], a["kk"], a["idx"], a["vals"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kk=0), 1), (dict(kk=2049), 2), (dict(fmt=3), 1), (dict(idx=None), 1),
    (dict(qrs=32 * 64 + 8), 3), (dict(T=0), 0),
    # the kept-score buffer of 600 rows x 32768 columns (8 bytes each) exceeds the
    # static scratch: refused before anything is enqueued
    (dict(T=600, out_cols=32768), 5),
])
def test_logits_topk_noalloc_argument_errors(kw, code):
    assert _noalloc(**kw) == code
    if code == 5:
        L = _lib.lib()
        need = L.fp4idx_logits_topk_workspace_bytes(0, kw["T"], 1, 32, 1, 64, 4, kw["out_cols"], 16)
        assert need > (128 << 20)
