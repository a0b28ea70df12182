"""ctypes front end of the CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It loads ``libfp4idx_oracle.so`` (built from
``fp4idx_oracle.c`` by ``build_oracle.py``), takes host numpy arrays and returns host
numpy arrays.  Nothing here touches a GPU or the GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build_oracle

MXFP4 = 0
NVFP4 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        # FP4IDX_ORACLE_LIB points at another build of the same source (used to check
        # that the pins catch planted mistakes in a modified copy of the oracle)
        path = os.environ.get("FP4IDX_ORACLE_LIB", build_oracle.LIB)
        if path == build_oracle.LIB and (
                not os.path.exists(path)
                or os.path.getmtime(path) < os.path.getmtime(build_oracle.SRC)):
            build_oracle.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.orc_e2m1.restype = ctypes.c_double
        L.orc_e2m1.argtypes = [ctypes.c_uint]
        L.orc_e8m0.restype = ctypes.c_double
        L.orc_e8m0.argtypes = [ctypes.c_uint]
        L.orc_e4m3.restype = ctypes.c_double
        L.orc_e4m3.argtypes = [ctypes.c_uint]
        L.orc_groups.restype = i32
        L.orc_groups.argtypes = [i32]
        L.orc_dequant_vec.restype = None
        L.orc_dequant_vec.argtypes = [i32, P, P, P]
        L.orc_dot.restype = i32
        L.orc_dot.argtypes = [P, P, P, P]
        L.orc_logits_paged.restype = ctypes.c_long
        L.orc_logits_paged.argtypes = [i32, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64,
                                       P, P, i32, i32, i32, i32, i32, i32, i32, i32, P, i64, P,
                                       P, i32, i32]
        L.orc_block_scores.restype = ctypes.c_long
        L.orc_block_scores.argtypes = [i32, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                       i32, i32, P, P, P, i32, i32]
        L.orc_topk.restype = None
        L.orc_topk.argtypes = [P, i64, i32, i32, P, i32, P, P, i32]
        L.orc_max_threads.restype = i32
        L.orc_max_threads.argtypes = [i32]
        L.orc_quantize_mx_block.restype = None
        L.orc_quantize_mx_block.argtypes = [P, P, P]
        L.orc_quantize_store.restype = None
        L.orc_quantize_store.argtypes = [P, P, i32, P, i64, P, i64, i32, i32]
        L.orc_qsa_offset_bits.restype = i32
        L.orc_qsa_offset_bits.argtypes = [i32]
        L.orc_qsa_slots.restype = None
        L.orc_qsa_slots.argtypes = [P, i64, i32, i32, P, i64, i32, i32, P, i32, i32, P, i64,
                                    i32]
        L.orc_qsa_decode.restype = None
        L.orc_qsa_decode.argtypes = [P, i64, i64, P, P, i64, i64, i64, i64, P, i64, P, i64,
                                     i32, i32, i32, i32, i32, i32, ctypes.c_double,
                                     ctypes.c_double, P, i64, i64, P, P, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def e8m0(code: int) -> float:
    return lib().orc_e8m0(code)


def e4m3(code: int) -> float:
    return lib().orc_e4m3(code)


def groups(fmt: int) -> int:
    return 4 if fmt == MXFP4 else 8


def dequant(fmt: int, packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., 64] packed codes + [..., G] scale codes -> [..., 128] float64 values."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    lead = packed.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    pk = packed.reshape(n, 64)
    sc = scales.reshape(n, groups(fmt))
    out = np.empty((n, 128), np.float64)
    L = lib()
    for i in range(n):
        L.orc_dequant_vec(fmt, _p(pk[i]), _p(sc[i]), _p(out[i]))
    return out.reshape(*lead, 128)


def dot(q: np.ndarray, k: np.ndarray):
    """Exact dot of two float64 128-vectors -> (value, provably_exact, sum |q_d k_d|)."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    out = np.zeros(1, np.float64)
    a = np.zeros(1, np.float64)
    ok = lib().orc_dot(_p(q), _p(k), _p(out), _p(a))
    return float(out[0]), bool(ok), float(a[0])


def logits_paged(fmt, q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens,
                 page_size, out_cols, num_pages=None, rows=None, n_threads=0,
                 want_tolbase=False, compact=False):
    """Weighted-ReLU logits.  Returns (logits [T,out_cols] float32 (only requested rows
    filled; others NaN), tolbase or None, number of inexact dots).

    compact=True (with rows): the result holds only the requested rows, in increasing
    row order ([len(rows), out_cols]); the call then sees just those rows, each still in
    its own request (cu_seqlens_q is recounted), which changes nothing they compute."""
    if compact and rows is not None:
        rows = np.unique(np.asarray(rows, np.int64))
        cu = np.asarray(cu_seqlens_q, np.int64)
        assert rows.size and rows[0] >= 0 and rows[-1] < cu[-1]
        b_of = np.searchsorted(cu, rows, side="right") - 1
        new_cu = np.zeros(cu.size, np.int32)
        new_cu[1:] = np.cumsum(np.bincount(b_of, minlength=cu.size - 1))
        return logits_paged(fmt, np.asarray(q_fp4)[rows], np.asarray(q_scale)[rows],
                            np.asarray(w)[rows], k_fp4, k_scale, block_table, new_cu,
                            np.asarray(row_lens)[rows], page_size, out_cols,
                            num_pages=num_pages, n_threads=n_threads, want_tolbase=want_tolbase)
    q_fp4 = _c(q_fp4, np.uint8)
    q_scale = _c(q_scale, np.uint8)
    w = _c(w, np.float32)
    k_fp4 = _c(k_fp4, np.uint8)
    k_scale = _c(k_scale, np.uint8)
    block_table = _c(block_table, np.int32)
    cu_seqlens_q = _c(cu_seqlens_q, np.int32)
    row_lens = _c(row_lens, np.int32)
    T, H = q_fp4.shape[0], q_fp4.shape[1]
    P, Hkv, page = k_fp4.shape[0], k_fp4.shape[1], k_fp4.shape[2]
    assert page == page_size
    G = groups(fmt)
    B, W = block_table.shape
    if num_pages is None:
        num_pages = P
    out = np.full((T, out_cols), np.nan, np.float32)
    tb = np.full((T, out_cols), np.nan, np.float32) if want_tolbase else None
    rows_a = None if rows is None else _c(rows, np.int32)
    n_rows = 0 if rows_a is None else int(rows_a.size)
    inexact = lib().orc_logits_paged(
        fmt, _p(q_fp4), H * 64, _p(q_scale), H * G, _p(w), H,
        _p(k_fp4), Hkv * page * 64, _p(k_scale), Hkv * page * G,
        _p(block_table), W, _p(cu_seqlens_q), _p(row_lens),
        T, B, H, Hkv, page, num_pages, W, out_cols, _p(out), out_cols, _p(tb),
        _p(rows_a), n_rows, n_threads)
    return out, tb, int(inexact)


def block_scores(fmt, q_fp4, q_scale, k_fp4, k_scale, cu_seqlens_q, cu_seqlens_k,
                 cu_page_offsets, kv_indices, qo_offset, max_seqlen_k, causal,
                 num_pages=None, rows=None, n_threads=0, want_errbase=False):
    """Per-head 128-block max scores [Hq, Ktiles, Tq] float32 (only requested query
    columns filled; others NaN), errbase or None, number of inexact dots."""
    q_fp4 = _c(q_fp4, np.uint8)
    q_scale = _c(q_scale, np.uint8)
    k_fp4 = _c(k_fp4, np.uint8)
    k_scale = _c(k_scale, np.uint8)
    cu_seqlens_q = _c(cu_seqlens_q, np.int32)
    cu_seqlens_k = _c(cu_seqlens_k, np.int32)
    cu_page_offsets = _c(cu_page_offsets, np.int32)
    kv_indices = _c(kv_indices, np.int32)
    qo = None if qo_offset is None else _c(qo_offset, np.int32)
    Tq, Hq = q_fp4.shape[0], q_fp4.shape[1]
    P, Hkv = k_fp4.shape[0], k_fp4.shape[1]
    assert k_fp4.shape[2] == 128
    B = cu_seqlens_q.size - 1
    if num_pages is None:
        num_pages = P
    ktiles = (max_seqlen_k + 127) // 128
    out = np.full((Hq, ktiles, Tq), np.nan, np.float32)
    eb = np.full((Hq, ktiles, Tq), np.nan, np.float32) if want_errbase else None
    rows_a = None if rows is None else _c(rows, np.int32)
    n_rows = 0 if rows_a is None else int(rows_a.size)
    inexact = lib().orc_block_scores(
        fmt, _p(q_fp4), _p(q_scale), _p(k_fp4), _p(k_scale), _p(cu_seqlens_q),
        _p(cu_seqlens_k), _p(cu_page_offsets), _p(kv_indices), _p(qo), B, Tq, Hq, Hkv,
        num_pages, max_seqlen_k, 1 if causal else 0, _p(out), _p(eb), _p(rows_a), n_rows,
        n_threads)
    return out, eb, int(inexact)


def topk(scores, k, row_lens=None, n_threads=0):
    """-> (idx [rows,k] int32 in increasing column order, -1 padded; vals [rows,k])."""
    scores = _c(scores, np.float32)
    rows, cols = scores.shape
    rl = None if row_lens is None else _c(row_lens, np.int32)
    idx = np.empty((rows, k), np.int32)
    vals = np.empty((rows, k), np.float32)
    lib().orc_topk(_p(scores), cols, rows, cols, _p(rl), k, _p(idx), _p(vals), n_threads)
    return idx, vals


def block_topk(scores, k, n_threads=0):
    """Top-k 128-token blocks of each (head, query) from block scores [Hq, Ktiles, Tq].

    [M3] The block-score interface returns scores only; a caller that wants TopK takes
    it along the Ktiles dimension (dim 1).  This is that TopK, with the same rule as
    ``topk``: the k largest finite scores (-inf and NaN never chosen, ties to the
    smaller block), listed in increasing block order and -1 padded.  The number of
    chosen blocks per (head, query) is the sparse metadata a block-sparse consumer
    needs next to the list.
    -> (idx [Hq, Tq, k] int32, count [Hq, Tq] int32)."""
    scores = _c(scores, np.float32)
    Hq, Kt, Tq = scores.shape
    rows = np.ascontiguousarray(np.transpose(scores, (0, 2, 1))).reshape(Hq * Tq, Kt)
    idx, _ = topk(rows, k, None, n_threads)
    idx = idx.reshape(Hq, Tq, k)
    count = (idx >= 0).sum(axis=2).astype(np.int32)
    return idx, count


def max_threads(n_threads=0) -> int:
    return int(lib().orc_max_threads(n_threads))


def quantize_mx_block(x):
    """32 real values -> (16 packed bytes, E8M0 code)."""
    x = _c(x, np.float64)
    assert x.shape == (32,)
    packed = np.zeros(16, np.uint8)
    code = np.zeros(1, np.uint8)
    lib().orc_quantize_mx_block(_p(x), _p(packed), _p(code))
    return packed, int(code[0])


def quantize_store(keys, slots, k_fp4, k_scale):
    """Keys [N,128] (real values) into copies of the cache arrays k_fp4 [P,1,page,64] and
    k_scale [P,1,page,4] at the given slots (others untouched) -> (k_fp4, k_scale)."""
    keys = _c(keys, np.float64)
    slots = _c(slots, np.int64)
    kf = np.array(k_fp4, dtype=np.uint8, copy=True, order="C")
    ks = np.array(k_scale, dtype=np.uint8, copy=True, order="C")
    P, hkv, page = kf.shape[0], kf.shape[1], kf.shape[2]
    assert hkv == 1 and ks.shape == (P, 1, page, 4) and keys.shape[1] == 128
    lib().orc_quantize_store(_p(keys), _p(slots), keys.shape[0], _p(kf), page * 64, _p(ks),
                             page * 4, page, P)
    return kf, ks


def qsa_offset_bits(page_size: int) -> int:
    """Bits of a slot that hold the place inside a page ([QSA] _decode_slot_layout)."""
    return int(lib().orc_qsa_offset_bits(page_size))


def qsa_slots(indices, block_table, token_to_req, num_cache_blocks, page_size, slot_cols=None):
    """[QSA] slot pass.  indices [rows, topk + 1] int32 (the last column is the valid
    count, not read here), block_table [num_requests, width] int32, token_to_req [rows]
    int32 -> slots [rows, slot_cols] int32 (slot_cols defaults to topk)."""
    ind = _c(indices, np.int32)
    bt = _c(block_table, np.int32)
    t2r = _c(token_to_req, np.int32)
    rows, topk = ind.shape[0], ind.shape[1] - 1
    slot_cols = topk if slot_cols is None else slot_cols
    out = np.empty((rows, slot_cols), np.int32)
    lib().orc_qsa_slots(_p(ind), ind.shape[1], rows, topk, _p(bt), bt.shape[1], bt.shape[0],
                        bt.shape[1], _p(t2r), num_cache_blocks, page_size, _p(out), slot_cols,
                        slot_cols)
    return out


def qsa_decode(q_bits, k_cache, v_cache, slots, indices, offset_bits, softmax_scale,
               output_scale, gate_bits, rows=None, n_threads=0, want_tolbase=False):
    """[QSA] sparse decode step in double.

    q_bits, gate_bits: [R, Hq, D] uint16 bf16 bit patterns.  k_cache, v_cache:
    [num_blocks, page, Hkv, D] uint8 e4m3fn codes (any byte strides; numpy views of one
    combined cache are fine).  slots [R, >= topk] int32, indices [R, topk + 1] int32.
    rows: optional subset of row ids (the result then holds just those rows, in the
    given order).  -> (out [n, Hq, D] float64, tolbase or None)."""
    q = np.asarray(q_bits)
    g = np.asarray(gate_bits)
    sl = np.asarray(slots)
    ind = np.asarray(indices)
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        q, g, sl, ind = q[rows], g[rows], sl[rows], ind[rows]
    q = _c(q, np.uint16)
    g = _c(g, np.uint16)
    sl = _c(sl, np.int32)
    ind = _c(ind, np.int32)
    kc = np.asarray(k_cache)
    vc = np.asarray(v_cache)
    assert kc.dtype == np.uint8 and vc.dtype == np.uint8
    assert kc.strides[3] == 1 and vc.strides[3] == 1 and kc.strides[:2] == vc.strides[:2]
    n, Hq, D = q.shape
    Hkv = kc.shape[2]
    topk = ind.shape[1] - 1
    out = np.zeros((n, Hq, D), np.float64)
    tb = np.zeros((n, Hq, D), np.float64) if want_tolbase else None
    lib().orc_qsa_decode(_p(q), Hq * D, D, kc.ctypes.data, vc.ctypes.data, kc.strides[0],
                         kc.strides[1], kc.strides[2], vc.strides[2], _p(sl), sl.shape[1],
                         _p(ind), ind.shape[1], topk, n, Hq, Hkv, D, offset_bits,
                         float(softmax_scale), float(output_scale), _p(g), Hq * D, D,
                         _p(out), _p(tb), n_threads)
    return out, tb
