"""sparse_attention_fp4_amd -- FP4 lightning-indexer scorer for MI355X (gfx950).

The compute path lives in libfp4idx.so (HIP kernels + the C ABI of include/fp4idx.h);
this package is its Python binding:

    logits_paged(...)   weighted-ReLU logits over a paged FP4 key cache
    logits_topk_paged(...)  their top-k without writing the logits (fused)
    logits_topk_paged_noalloc(...)  the same without a workspace (static per-GPU scratch)
    block_scores(...)   per-head 128-token block-max scores
    block_topk(...)     top-k blocks per (head, query) along the block scores' Ktiles
    topk(...)           exact top-k column selection per row
    quantize_store_k(...)  MXFP4 quantize-and-store of keys into the paged cache
    qsa_sparse_paged_decode(...)  sparse attention over the selected tokens of an fp8
                        K/V cache (slot pass ``qsa_slots`` + ``qsa_decode``)

``workloads`` holds seeded synthetic inputs for the benchmark shapes.
"""
from .ops import (MXFP4, NVFP4, block_scores, block_topk, logits_paged,  # noqa: F401
                  logits_topk_paged, logits_topk_paged_noalloc, logits_topk_workspace_bytes,
                  qsa_decode, qsa_slots, qsa_sparse_paged_decode, quantize_store_k, topk,
                  topk_workspace_bytes)

__all__ = ["MXFP4", "NVFP4", "logits_paged", "logits_topk_paged", "logits_topk_paged_noalloc",
           "logits_topk_workspace_bytes", "block_scores", "block_topk", "topk",
           "topk_workspace_bytes", "quantize_store_k", "qsa_slots", "qsa_decode",
           "qsa_sparse_paged_decode"]
