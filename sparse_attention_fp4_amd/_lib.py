"""Loader of libfp4idx.so, the C ABI declared in include/fp4idx.h.

The library is built in-tree by ``sparse_attention_fp4_amd/build.py`` (or
``__graft_entry__.build()``).  Loading never falls back to anything else: if the
shared object is missing the import of the op layer raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4idx.so")

# the symbols include/fp4idx.h declares
EXPORTS = (
    "fp4idx_logits_paged",
    "fp4idx_logits_topk_workspace_bytes",
    "fp4idx_logits_topk_paged",
    "fp4idx_logits_topk_paged_noalloc",
    "fp4idx_block_scores",
    "fp4idx_block_topk",
    "fp4idx_topk_workspace_bytes",
    "fp4idx_topk",
    "fp4idx_set_topk_wait_limit",
    "fp4idx_quantize_store_k",
    "fp4idx_qsa_slots",
    "fp4idx_qsa_decode",
    "fp4idx_strerror",
    "fp4idx_version",
)

_lib = None


class Fp4idxError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = lib().fp4idx_strerror(code).decode()
        super().__init__(f"{fn} failed: {msg} (status {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sparse_attention_fp4_amd/build.py` "
            "(the FP4 indexer has no other implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.fp4idx_logits_paged.restype = i32
    L.fp4idx_logits_paged.argtypes = [i32, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P, P,
                                      i32, i32, i32, i32, i32, i32, i32, i32, P, i64, P]
    L.fp4idx_logits_topk_workspace_bytes.restype = ctypes.c_size_t
    L.fp4idx_logits_topk_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32]
    L.fp4idx_logits_topk_paged.restype = i32
    L.fp4idx_logits_topk_paged.argtypes = [i32, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P,
                                           P, i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P,
                                           P, ctypes.c_size_t, P]
    L.fp4idx_logits_topk_paged_noalloc.restype = i32
    L.fp4idx_logits_topk_paged_noalloc.argtypes = [i32, P, i64, P, i64, P, i64, P, i64, P, i64, P,
                                                   i64, P, P, i32, i32, i32, i32, i32, i32, i32,
                                                   i32, i32, P, P, P]
    L.fp4idx_block_scores.restype = i32
    L.fp4idx_block_scores.argtypes = [i32, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                      i32, i32, i32, P, P]
    L.fp4idx_block_topk.restype = i32
    L.fp4idx_block_topk.argtypes = [P, i32, i32, i32, i32, P, P, P]
    L.fp4idx_topk_workspace_bytes.restype = ctypes.c_size_t
    L.fp4idx_topk_workspace_bytes.argtypes = [i32, i32, i32]
    L.fp4idx_topk.restype = i32
    L.fp4idx_topk.argtypes = [P, i64, i32, i32, P, i32, P, P, P, ctypes.c_size_t, P]
    L.fp4idx_set_topk_wait_limit.restype = i32
    L.fp4idx_set_topk_wait_limit.argtypes = [i32]
    L.fp4idx_quantize_store_k.restype = i32
    L.fp4idx_quantize_store_k.argtypes = [P, i64, P, i32, P, i64, P, i64, i32, i32, P]
    L.fp4idx_qsa_slots.restype = i32
    L.fp4idx_qsa_slots.argtypes = [P, i64, i32, i32, P, i64, i32, i32, P, i32, i32, P, i64, i32,
                                   P]
    f32 = ctypes.c_float
    L.fp4idx_qsa_decode.restype = i32
    L.fp4idx_qsa_decode.argtypes = [P, i64, i64, P, P, i64, i64, i64, i64, i32, i32, P, i64, P,
                                    i64, i32, i32, i32, i32, i32, f32, f32, P, i64, i64, P, i64,
                                    i64, P]
    L.fp4idx_strerror.restype = ctypes.c_char_p
    L.fp4idx_strerror.argtypes = [i32]
    L.fp4idx_version.restype = i32
    L.fp4idx_version.argtypes = []
    _lib = L
    return L


def check(fn: str, code: int) -> None:
    if code != 0:
        raise Fp4idxError(fn, code)
