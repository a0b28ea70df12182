"""Python binding of the FP4 indexer C ABI (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks dtypes,
shapes and devices on the host, and calls the matching ``fp4idx_*`` entry point of
libfp4idx.so on torch's current HIP stream.  All arithmetic happens in the library's
HIP kernels; nothing here computes a score.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import check, lib

MXFP4 = 0
NVFP4 = 1
_FMT = {"mxfp4": MXFP4, "nvfp4": NVFP4, MXFP4: MXFP4, NVFP4: NVFP4}


def _fmt(fmt) -> int:
    try:
        return _FMT[fmt]
    except KeyError:
        raise ValueError(f"unknown FP4 format {fmt!r}") from None


def _groups(fmt: int) -> int:
    return 4 if fmt == MXFP4 else 8


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _u8(t):
    """Packed codes may arrive as uint8, int8 or a 1-byte float view: read as bytes."""
    if t.dtype == torch.uint8:
        return t
    if t.element_size() == 1:
        return t.view(torch.uint8)
    raise ValueError(f"expected a 1-byte dtype, got {t.dtype}")


def _logits_args(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens, fmt,
                 k_page_stride, ks_page_stride):
    """Checked tensors and the scalar arguments shared by the logits entry points."""
    f = _fmt(fmt)
    G = _groups(f)
    q_fp4, q_scale, k_fp4, k_scale = _u8(q_fp4), _u8(q_scale), _u8(k_fp4), _u8(k_scale)
    dev = q_fp4.device
    _need(q_fp4, "q_fp4", torch.uint8, 3, dev)
    _need(q_scale, "q_scale", torch.uint8, 3, dev)
    _need(w, "w", torch.float32, 2, dev)
    _need(k_fp4, "k_fp4", torch.uint8, 4, dev)
    _need(k_scale, "k_scale", torch.uint8, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _need(row_lens, "row_lens", torch.int32, 1, dev)
    T, H, d2 = q_fp4.shape
    P, Hkv, page, d2k = k_fp4.shape
    if d2 != 64 or d2k != 64:
        raise ValueError("q_fp4 / k_fp4 must pack D=128 as 64 bytes")
    if q_scale.shape != (T, H, G) or w.shape != (T, H):
        raise ValueError("q_scale must be [T,H,G] and w [T,H]")
    if k_scale.shape != (P, Hkv, page, G):
        raise ValueError("k_scale must be [P,Hkv,page,G]")
    B, W = block_table.shape
    if cu_seqlens_q.numel() != B + 1 or row_lens.numel() != T:
        raise ValueError("cu_seqlens_q must have B+1 entries and row_lens T")
    for name, t in (("q_fp4", q_fp4), ("q_scale", q_scale), ("w", w)):
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != t.shape[2]):
            raise ValueError(f"{name} must be contiguous within a row")
    for name, t, width in (("k_fp4", k_fp4, 64), ("k_scale", k_scale, G)):
        if t.stride(3) != 1 or t.stride(2) != width or t.stride(1) != page * width:
            raise ValueError(f"{name} must be contiguous inside each page")
    if block_table.stride(1) != 1 or not cu_seqlens_q.is_contiguous() or not row_lens.is_contiguous():
        raise ValueError("metadata tensors must be contiguous")
    kps = k_page_stride if k_page_stride is not None else (k_fp4.stride(0) if P > 0 else Hkv * page * 64)
    ksps = ks_page_stride if ks_page_stride is not None else (k_scale.stride(0) if P > 0 else Hkv * page * G)
    args = (f, _ptr(q_fp4), q_fp4.stride(0), _ptr(q_scale), q_scale.stride(0), _ptr(w), w.stride(0),
            _ptr(k_fp4), kps, _ptr(k_scale), ksps, _ptr(block_table), block_table.stride(0),
            _ptr(cu_seqlens_q), _ptr(row_lens), T, B, H, Hkv, page, P, W)
    return args, dict(dev=dev, T=T, B=B, H=H, Hkv=Hkv, page=page, W=W, fmt=f)


def logits_paged(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens, *,
                 fmt="mxfp4", out_cols: int, out: Optional[torch.Tensor] = None,
                 k_page_stride: Optional[int] = None, ks_page_stride: Optional[int] = None):
    """Weighted-ReLU logits [T, out_cols] fp32 (-inf where invisible).

    q_fp4 [T,H,64] u8 (row stride may exceed H*64), q_scale [T,H,G] u8, w [T,H] fp32,
    k_fp4 [P,Hkv,page,64] u8, k_scale [P,Hkv,page,G] u8, block_table [B,W] int32,
    cu_seqlens_q [B+1] int32, row_lens [T] int32.
    """
    args, d = _logits_args(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens,
                           fmt, k_page_stride, ks_page_stride)
    T, dev = d["T"], d["dev"]
    if out is None:
        out = torch.empty((T, out_cols), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, 2, dev)
        if out.shape != (T, out_cols) or out.stride(1) != 1:
            raise ValueError("out must be [T, out_cols] with unit column stride")
    rc = lib().fp4idx_logits_paged(*args, out_cols, _ptr(out), out.stride(0), _stream())
    check("fp4idx_logits_paged", rc)
    return out


def logits_topk_workspace_bytes(fmt, T, B, H, Hkv, page_size, table_width, out_cols, k) -> int:
    return int(lib().fp4idx_logits_topk_workspace_bytes(_fmt(fmt), T, B, H, Hkv, page_size,
                                                        table_width, out_cols, k))


def logits_topk_paged(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens, *,
                      fmt="mxfp4", out_cols: int, k: int, out_idx=None, out_vals=None,
                      want_vals=True, workspace=None, k_page_stride: Optional[int] = None,
                      ks_page_stride: Optional[int] = None):
    """Top-k columns of the weighted-ReLU logits without writing the logits: exactly
    topk(logits_paged(...), k, row_lens) -> (idx [T, k] int32 in increasing column order,
    -1 padded; vals [T, k] fp32 or None).  workspace: optional uint8 device tensor of at
    least logits_topk_workspace_bytes(...) bytes (allocated when omitted)."""
    args, d = _logits_args(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens,
                           fmt, k_page_stride, ks_page_stride)
    T, dev = d["T"], d["dev"]
    if out_idx is None:
        out_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if out_vals is None and want_vals:
        out_vals = torch.empty((T, k), dtype=torch.float32, device=dev)
    for name, t, dt in (("out_idx", out_idx, torch.int32), ("out_vals", out_vals, torch.float32)):
        if t is not None:
            _need(t, name, dt, 2, dev)
            if t.shape != (T, k) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [T, k] tensor")
    need = logits_topk_workspace_bytes(d["fmt"], T, d["B"], d["H"], d["Hkv"], d["page"], d["W"],
                                       out_cols, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().fp4idx_logits_topk_paged(*args, out_cols, k, _ptr(out_idx), _ptr(out_vals),
                                        _ptr(workspace), ws_bytes, _stream())
    check("fp4idx_logits_topk_paged", rc)
    return out_idx, out_vals


def logits_topk_paged_noalloc(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q,
                              row_lens, *, fmt="mxfp4", out_cols: int, k: int, out_idx,
                              out_vals=None, k_page_stride: Optional[int] = None,
                              ks_page_stride: Optional[int] = None):
    """logits_topk_paged without a workspace: the library's per-GPU static scratch is used
    and nothing is allocated (out_idx, and out_vals if wanted, are the caller's)."""
    args, d = _logits_args(q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu_seqlens_q, row_lens,
                           fmt, k_page_stride, ks_page_stride)
    T, dev = d["T"], d["dev"]
    for name, t, dt in (("out_idx", out_idx, torch.int32), ("out_vals", out_vals, torch.float32)):
        if t is not None:
            _need(t, name, dt, 2, dev)
            if t.shape != (T, k) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [T, k] tensor")
    rc = lib().fp4idx_logits_topk_paged_noalloc(*args, out_cols, k, _ptr(out_idx), _ptr(out_vals),
                                                _stream())
    check("fp4idx_logits_topk_paged_noalloc", rc)
    return out_idx, out_vals


def block_scores(q_fp4, k_fp4, q_scale, k_scale, cu_seqlens_q, cu_seqlens_k, cu_page_offsets, *,
                 max_seqlen_q: int, max_seqlen_k: int, kv_indices, fmt="nvfp4", causal=True,
                 qo_offset=None, out: Optional[torch.Tensor] = None):
    """Per-head 128-token block-max scores [Hq, ceil(max_seqlen_k/128), Tq] fp32.

    Argument order follows the M3 README's public API."""
    f = _fmt(fmt)
    G = _groups(f)
    q_fp4, q_scale, k_fp4, k_scale = _u8(q_fp4), _u8(q_scale), _u8(k_fp4), _u8(k_scale)
    dev = q_fp4.device
    _need(q_fp4, "q_fp4", torch.uint8, 3, dev)
    _need(q_scale, "q_scale", torch.uint8, 3, dev)
    _need(k_fp4, "k_fp4", torch.uint8, 4, dev)
    _need(k_scale, "k_scale", torch.uint8, 4, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                    ("cu_page_offsets", cu_page_offsets), ("kv_indices", kv_indices)):
        _need(t, name, torch.int32, 1, dev)
    if qo_offset is not None:
        _need(qo_offset, "qo_offset", torch.int32, 1, dev)
        if not causal:
            raise ValueError("qo_offset is only allowed with causal=True")
    Tq, Hq, _ = q_fp4.shape
    P, Hkv, page, _ = k_fp4.shape
    if page != 128:
        raise ValueError("block scores need 128-token pages")
    if q_scale.shape != (Tq, Hq, G) or k_scale.shape != (P, Hkv, 128, G):
        raise ValueError("scale shapes must be [Tq,Hq,G] and [P,Hkv,128,G]")
    for name, t in (("q_fp4", q_fp4), ("q_scale", q_scale), ("k_fp4", k_fp4), ("k_scale", k_scale),
                    ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                    ("cu_page_offsets", cu_page_offsets), ("kv_indices", kv_indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B = cu_seqlens_q.numel() - 1
    ktiles = (max_seqlen_k + 127) // 128
    if out is None:
        out = torch.empty((Hq, ktiles, Tq), dtype=torch.float32, device=dev)
    elif out.shape != (Hq, ktiles, Tq) or not out.is_contiguous():
        raise ValueError("out must be contiguous [Hq, Ktiles, Tq]")
    rc = lib().fp4idx_block_scores(
        f, _ptr(q_fp4), _ptr(q_scale), _ptr(k_fp4), _ptr(k_scale), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), _ptr(cu_page_offsets), _ptr(kv_indices), _ptr(qo_offset),
        B, Tq, Hq, Hkv, P, max_seqlen_q, max_seqlen_k, 1 if causal else 0, _ptr(out), _stream())
    check("fp4idx_block_scores", rc)
    return out


def topk_workspace_bytes(rows: int, cols: int, k: int) -> int:
    return int(lib().fp4idx_topk_workspace_bytes(rows, cols, k))


def topk(scores, k: int, row_lens=None, *, out_idx=None, out_vals=None, want_vals=True,
         workspace=None):
    """Top-k columns per row in increasing column order, -1 padded -> (idx, vals|None).

    workspace: optional uint8 tensor of at least topk_workspace_bytes(rows, cols, k)
    bytes, zero-filled before its first use (torch.zeros); each call leaves it ready for
    the next one of the same rows and cols, so it can be reused across such calls
    without clearing (zero it again before a call of another shape).
    """
    _need(scores, "scores", torch.float32, 2)
    dev = scores.device
    rows, cols = scores.shape
    if scores.stride(1) != 1:
        raise ValueError("scores must have unit column stride")
    if row_lens is not None:
        _need(row_lens, "row_lens", torch.int32, 1, dev)
        if row_lens.numel() != rows or not row_lens.is_contiguous():
            raise ValueError("row_lens must be a contiguous [rows] tensor")
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if want_vals and out_vals is None:
        out_vals = torch.empty((rows, k), dtype=torch.float32, device=dev)
    need = topk_workspace_bytes(rows, cols, k)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)  # zero before first use
    rc = lib().fp4idx_topk(_ptr(scores), scores.stride(0), rows, cols, _ptr(row_lens), k,
                           _ptr(out_idx), _ptr(out_vals), _ptr(workspace),
                           0 if workspace is None else workspace.numel(), _stream())
    check("fp4idx_topk", rc)
    return out_idx, out_vals


def set_topk_wait_limit(polls: int) -> int:
    """Bound on each in-kernel wait of the few-long-rows top-k (0 forces its fallback,
    where one workgroup recomputes a row); returns the previous bound."""
    return int(lib().fp4idx_set_topk_wait_limit(int(polls)))


def block_topk(scores, k: int, *, out_idx=None, out_count=None):
    """Top-k 128-token blocks per (head, query) along Ktiles of block scores
    [Hq, Ktiles, Tq] -> (idx [Hq, Tq, k] int32 in increasing block order, -1 padded,
    count [Hq, Tq] int32)."""
    _need(scores, "scores", torch.float32, 3)
    if not scores.is_contiguous():
        raise ValueError("scores must be contiguous [Hq, Ktiles, Tq]")
    dev = scores.device
    Hq, Kt, Tq = scores.shape
    if out_idx is None:
        out_idx = torch.empty((Hq, Tq, k), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((Hq, Tq), dtype=torch.int32, device=dev)
    rc = lib().fp4idx_block_topk(_ptr(scores), Hq, Kt, Tq, k, _ptr(out_idx), _ptr(out_count),
                                 _stream())
    check("fp4idx_block_topk", rc)
    return out_idx, out_count


def quantize_store_k(keys, slots, k_fp4, k_scale):
    """MXFP4 quantize-and-store of keys [N, 128] (bf16) into the paged cache k_fp4
    [P, 1, page, 64] / k_scale [P, 1, page, 4] (uint8, modified in place) at the given
    slots [N] (int64; slots outside the cache are skipped)."""
    _need(keys, "keys", torch.bfloat16, 2)
    dev = keys.device
    k_fp4, k_scale = _u8(k_fp4), _u8(k_scale)
    _need(slots, "slots", torch.int64, 1, dev)
    _need(k_fp4, "k_fp4", torch.uint8, 4, dev)
    _need(k_scale, "k_scale", torch.uint8, 4, dev)
    N, D = keys.shape
    P, hkv, page, _ = k_fp4.shape
    if D != 128 or keys.stride(1) != 1:
        raise ValueError("keys must be [N, 128] with unit column stride")
    if hkv != 1 or k_fp4.shape != (P, 1, page, 64) or k_scale.shape != (P, 1, page, 4):
        raise ValueError("cache must be k_fp4 [P,1,page,64] and k_scale [P,1,page,4]")
    if slots.numel() != N or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous [N] tensor")
    if not (k_fp4.is_contiguous() and k_scale.is_contiguous()):
        raise ValueError("cache tensors must be contiguous")
    rc = lib().fp4idx_quantize_store_k(_ptr(keys), keys.stride(0), _ptr(slots), N, _ptr(k_fp4),
                                       page * 64, _ptr(k_scale), page * 4, page, P, _stream())
    check("fp4idx_quantize_store_k", rc)
    return k_fp4, k_scale


def qsa_slots(logical_indices, block_table, token_to_req, num_cache_blocks: int, page_size: int,
              *, out=None, slot_cols: Optional[int] = None):
    """Slot pass of the sparse attention over selected tokens (vLLM qsa_fp8 page,
    _qsa_physical_slots_kernel): logical_indices [rows, topk + 1] int32 (the valid count
    in the last column), block_table [num_requests, width] int32, token_to_req [rows]
    int32 -> slots [rows, slot_cols] int32, (page << offset_bits) | place or -1."""
    _need(logical_indices, "logical_indices", torch.int32, 2)
    dev = logical_indices.device
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(token_to_req, "token_to_req", torch.int32, 1, dev)
    rows, cols = logical_indices.shape
    topk = cols - 1
    slot_cols = topk if slot_cols is None else int(slot_cols)
    for t, name in ((logical_indices, "logical_indices"), (block_table, "block_table")):
        if t.stride(1) != 1:
            raise ValueError(f"{name} must have unit column stride")
    if token_to_req.numel() != rows or not token_to_req.is_contiguous():
        raise ValueError("token_to_req must be a contiguous [rows] tensor")
    if out is None:
        out = torch.empty((rows, slot_cols), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, 2, dev)
    if out.stride(1) != 1 or out.shape != (rows, slot_cols):
        raise ValueError("out must be [rows, slot_cols] with unit column stride")
    rc = lib().fp4idx_qsa_slots(_ptr(logical_indices), logical_indices.stride(0), rows, topk,
                                _ptr(block_table), block_table.stride(0), block_table.shape[0],
                                block_table.shape[1], _ptr(token_to_req), num_cache_blocks,
                                page_size, _ptr(out), out.stride(0), slot_cols, _stream())
    check("fp4idx_qsa_slots", rc)
    return out


def _cache_view(t, name):
    t = _u8(t)
    _need(t, name, torch.uint8, 4)
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have contiguous head dims")
    return t


def qsa_decode(q, k_cache, v_cache, slots, logical_indices, out, output_gate,
               softmax_scale: float, output_scale: float):
    """Sparse grouped-query attention over the selected tokens (vLLM qsa_fp8 page,
    _qsa_sparse_paged_decode_kernel) given the slots of ``qsa_slots``.
    q, output_gate, out: [rows, Hq, 128] bf16; k_cache, v_cache: [num_blocks, page, Hkv,
    128] e4m3fn codes (uint8 or float8_e4m3fn views, equal block and token strides)."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    k_cache, v_cache = _cache_view(k_cache, "k_cache"), _cache_view(v_cache, "v_cache")
    _need(slots, "slots", torch.int32, 2, dev)
    _need(logical_indices, "logical_indices", torch.int32, 2, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(output_gate, "output_gate", torch.bfloat16, 3, dev)
    rows, Hq, D = q.shape
    nb, page, Hkv, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.stride()[:2] != k_cache.stride()[:2]:
        raise ValueError("k_cache and v_cache must have the same shape and block/token strides")
    if Dk != D or out.shape != q.shape or output_gate.shape != q.shape:
        raise ValueError("q, out, output_gate must be [rows, Hq, D] with the cache's D")
    for t, name in ((q, "q"), (out, "out"), (output_gate, "output_gate")):
        if t.stride(2) != 1:
            raise ValueError(f"{name} must have unit dim stride")
    if slots.shape[0] != rows or slots.stride(1) != 1 or logical_indices.shape[0] != rows \
            or logical_indices.stride(1) != 1:
        raise ValueError("slots and logical_indices must have one row per query row")
    topk = logical_indices.shape[1] - 1
    if slots.shape[1] < topk:
        raise ValueError("slots must have at least topk columns")
    rc = lib().fp4idx_qsa_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), _ptr(v_cache), k_cache.stride(0),
        k_cache.stride(1), k_cache.stride(2), v_cache.stride(2), nb, page, _ptr(slots),
        slots.stride(0), _ptr(logical_indices), logical_indices.stride(0), topk, rows, Hq, Hkv,
        D, float(softmax_scale), float(output_scale), _ptr(output_gate), output_gate.stride(0),
        output_gate.stride(1), _ptr(out), out.stride(0), out.stride(1), _stream())
    check("fp4idx_qsa_decode", rc)
    return out


def qsa_sparse_paged_decode(q, k_cache, v_cache, logical_indices, block_table, token_to_req,
                            out, output_gate, softmax_scale: float, output_scale: float,
                            *, slots=None):
    """The slot pass then the sparse decode (vLLM qsa_fp8 page, qsa_sparse_paged_decode).
    slots: optional preallocated [rows, >= topk] int32 buffer."""
    k8 = _cache_view(k_cache, "k_cache")
    rows = q.shape[0]
    topk = logical_indices.shape[1] - 1
    if slots is None:
        slots = torch.empty((rows, topk), dtype=torch.int32, device=q.device)
    qsa_slots(logical_indices, block_table, token_to_req, k8.shape[0], k8.shape[1], out=slots,
              slot_cols=slots.shape[1])
    return qsa_decode(q, k_cache, v_cache, slots, logical_indices, out, output_gate,
                      softmax_scale, output_scale)
