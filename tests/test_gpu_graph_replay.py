"""Calls captured in a HIP graph, replayed after their metadata changed in place.

"[DSv4.1] Speed up the FP4 indexer scorer..." (Accuracy Tests: graph replay must pick up
new visibility and a new page mapping; the paged logits under replay).  The entry
points read every length, offset and table on the device when their kernels run, so a
captured call replayed after the caller rewrote `row_lens`, `block_table`,
`cu_seqlens_*`, `cu_page_offsets`, `kv_indices` or `qo_offset` in the same buffers must
compute what an eager call on the new metadata computes.  Each variant below is
replayed twice (the long-row top-k's workspace must be left ready by every replay), with
eager work and synchronisations between replays; every replay is compared with the
oracle on the new metadata and bit for bit with an eager call on separate buffers.
"""
import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import DOT_BOUND, check_logits, check_topk_against_oracle, dev, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Capture fn() into a graph on a side stream (one eager run first)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _logits_variants(case, rng, n):
    """n metadata variants of a logits case with the same shapes: new row lengths
    (0 and the full width included), a new split of the rows between the requests, and
    a new page mapping (any physical page, some -1 and some out-of-cache entries)."""
    B, W = case.block_table.shape
    T, P = case.T, case.num_pages
    out = []
    for v in range(n):
        bt = rng.integers(0, P, size=(B, W)).astype(np.int32)
        bt[rng.random((B, W)) < 0.05] = -1
        bt[rng.random((B, W)) < 0.02] = P + 7
        cuts = np.sort(rng.integers(0, T + 1, size=B - 1))
        cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
        lens = rng.integers(0, case.out_cols + 1, size=T).astype(np.int32)
        lens[v % T] = case.out_cols
        lens[(v + 1) % T] = 0
        out.append(dict(block_table=bt, cu_seqlens_q=cu, row_lens=lens))
    return out


def _with(case, meta):
    import copy
    c = copy.copy(case)
    for k_, v_ in meta.items():
        setattr(c, k_, v_)
    return c


@pytest.mark.parametrize("ctx0", [20000, 40000], ids=["one_kernel_topk", "three_kernel_topk"])
@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4], ids=["mxfp4", "nvfp4"])
def test_logits_and_long_row_topk_replay_with_new_visibility_and_mapping(fmt, ctx0):
    """5 rows of 20000 columns take the one-kernel long-row top-k (in-memory waits on
    counters it clears itself), 5 rows of 40000 the three kernels."""
    k = 2048
    case = wl.make_logits(f"replay_{fmt}_{ctx0}", fmt=fmt, q_per_req=[3, 2], ctx=[ctx0, 12000], H=32,
                          seed=211 + fmt)
    T, oc = case.T, case.out_cols
    q, qs, w, kf, ks = (dev(a) for a in (case.q_fp4, case.q_scale, case.w, case.k_fp4, case.k_scale))
    bt, cu, lens = dev(case.block_table), dev(case.cu_seqlens_q), dev(case.row_lens)
    out = torch.empty((T, oc), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((T, k), dtype=torch.float32, device="cuda")
    need = fp4.topk_workspace_bytes(T, oc, k)
    assert need > 0, "this shape is meant to take the long-row top-k (with a workspace)"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

    def calls():
        fp4.logits_paged(q, qs, w, kf, ks, bt, cu, lens, fmt=fmt, out_cols=oc, out=out)
        fp4.topk(out, k, lens, out_idx=idx, out_vals=vals, workspace=ws)

    g = _capture(calls)
    for v, meta in enumerate(_logits_variants(case, np.random.default_rng(5 + fmt), 3)):
        bt.copy_(torch.from_numpy(meta["block_table"]))
        cu.copy_(torch.from_numpy(meta["cu_seqlens_q"]))
        lens.copy_(torch.from_numpy(meta["row_lens"]))
        torch.cuda.synchronize()
        c = _with(case, meta)
        ref, tb, inexact = orc.logits_paged(c.fmt, c.q_fp4, c.q_scale, c.w, c.k_fp4, c.k_scale,
                                            c.block_table, c.cu_seqlens_q, c.row_lens,
                                            c.page_size, oc, want_tolbase=True)
        assert inexact == 0
        # eager reference on separate buffers
        e_out = fp4.logits_paged(q, qs, w, kf, ks, bt, cu, lens, fmt=fmt, out_cols=oc)
        e_idx, e_vals = fp4.topk(e_out, k, lens)
        torch.cuda.synchronize()
        e_out, e_idx, e_vals = e_out.cpu().numpy(), e_idx.cpu().numpy(), e_vals.cpu().numpy()
        for rep in range(2):
            say(f"[gpu] graph replay: logits + top-{k}, fmt={fmt}, ctx {ctx0}, variant {v}, replay {rep}")
            out.fill_(np.nan)
            idx.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got, gi, gv = out.cpu().numpy(), idx.cpu().numpy(), vals.cpu().numpy()
            check_logits(got, ref, tb)
            np.testing.assert_array_equal(got.view(np.uint32), e_out.view(np.uint32))
            np.testing.assert_array_equal(gi, e_idx)
            np.testing.assert_array_equal(gv.view(np.uint32), e_vals.view(np.uint32))
            # the top-k of the GPU's own scores equals the oracle's top-k of them exactly
            oi, _ = orc.topk(got, k, np.minimum(c.row_lens, oc))
            np.testing.assert_array_equal(gi, oi)
            nd = check_topk_against_oracle(ref, tb, gi, k, np.minimum(c.row_lens, oc))
            say(f"    ok (ties within tolerance against the oracle's logits: {nd})")


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4], ids=["mxfp4", "nvfp4"])
def test_block_scores_replay_with_new_lengths_pages_and_offsets(fmt):
    case = wl.make_block(f"breplay_{fmt}", fmt=fmt, q_lens=[20, 33, 11], k_lens=[300, 700, 129],
                         Hq=8, Hkv=2, seed=223 + fmt, causal=True, qo_offset=[280, 667, 118],
                         extra_pages=5)
    case.max_seqlen_q = 64
    case.max_seqlen_k = 1000
    P = case.k_fp4.shape[0]
    Tq = case.Tq
    q, qs, kf, ks = (dev(a) for a in (case.q_fp4, case.q_scale, case.k_fp4, case.k_scale))
    cuq, cuk = dev(case.cu_seqlens_q), dev(case.cu_seqlens_k)
    cup = dev(case.cu_page_offsets)
    kvi = torch.full((P,), -1, dtype=torch.int32, device="cuda")
    kvi[:case.kv_indices.size].copy_(torch.from_numpy(case.kv_indices))
    qo = dev(case.qo_offset)
    ktiles = (case.max_seqlen_k + 127) // 128
    out = torch.empty((case.Hq, ktiles, Tq), dtype=torch.float32, device="cuda")

    def call(o):
        return fp4.block_scores(q, kf, qs, ks, cuq, cuk, cup, max_seqlen_q=case.max_seqlen_q,
                                max_seqlen_k=case.max_seqlen_k, kv_indices=kvi, fmt=fmt,
                                causal=True, qo_offset=qo, out=o)

    g = _capture(lambda: call(out))
    rng = np.random.default_rng(17 + fmt)
    variants = [([30, 4, 30], [900, 64, 500], [870, 60, 470]),
                ([1, 62, 1], [1000, 128, 1], [999, -5, 0]),
                ([64, 0, 0], [257, 0, 0], [300, 0, 0])]
    for v, (ql, kl, off) in enumerate(variants):
        npg = [-(-x // 128) for x in kl]
        kv_new = np.full(P, -1, np.int32)
        kv_new[:sum(npg)] = rng.permutation(P)[:sum(npg)]
        if sum(npg) > 2:
            kv_new[1] = -1                                  # a hole
        meta = dict(cu_seqlens_q=np.concatenate([[0], np.cumsum(ql)]).astype(np.int32),
                    cu_seqlens_k=np.concatenate([[0], np.cumsum(kl)]).astype(np.int32),
                    cu_page_offsets=np.concatenate([[0], np.cumsum(npg)]).astype(np.int32),
                    kv_indices=kv_new, qo_offset=np.asarray(off, np.int32))
        cuq.copy_(torch.from_numpy(meta["cu_seqlens_q"]))
        cuk.copy_(torch.from_numpy(meta["cu_seqlens_k"]))
        cup.copy_(torch.from_numpy(meta["cu_page_offsets"]))
        kvi.copy_(torch.from_numpy(meta["kv_indices"]))
        qo.copy_(torch.from_numpy(meta["qo_offset"]))
        torch.cuda.synchronize()
        c = _with(case, meta)
        ref, eb, inexact = orc.block_scores(c.fmt, c.q_fp4, c.q_scale, c.k_fp4, c.k_scale,
                                            c.cu_seqlens_q, c.cu_seqlens_k, c.cu_page_offsets,
                                            c.kv_indices, c.qo_offset, c.max_seqlen_k, True,
                                            want_errbase=True)
        assert inexact == 0
        eager = call(torch.empty_like(out))
        torch.cuda.synchronize()
        eager = eager.cpu().numpy()
        for rep in range(2):
            say(f"[gpu] graph replay: block scores fmt={fmt}, variant {v}, replay {rep}")
            out.fill_(np.nan)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            np.testing.assert_array_equal(got.view(np.uint32), eager.view(np.uint32))
            # rows past cu_seqlens_q[B] are not written; compare the rows of the batch
            nq = int(meta["cu_seqlens_q"][-1])
            g_, r_, e_ = got[:, :, :nq], ref[:, :, :nq], eb[:, :, :nq]
            inv = r_ == -np.inf
            assert np.array_equal(g_ == -np.inf, inv)
            assert np.all(np.abs(g_[~inv].astype(np.float64) - r_[~inv]) <= DOT_BOUND[fmt] * e_[~inv])


@pytest.mark.parametrize("T,ctx,q_per_req,H", [
    (5, [20000, 12000], [3, 2], 32),           # fewer than 512 rows: logits in the workspace
    (560, [3000, 4100, 2500], [200, 250, 110], 8),   # 512 or more: sampled threshold
], ids=["few_rows", "many_rows"])
def test_fused_topk_replay_with_new_visibility_and_mapping(T, ctx, q_per_req, H):
    k = 2048 if T < 512 else 256
    case = wl.make_logits(f"freplay_{T}", q_per_req=q_per_req, ctx=ctx, H=H, seed=229 + T)
    oc = case.out_cols
    q, qs, w, kf, ks = (dev(a) for a in (case.q_fp4, case.q_scale, case.w, case.k_fp4, case.k_scale))
    bt, cu, lens = dev(case.block_table), dev(case.cu_seqlens_q), dev(case.row_lens)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((T, k), dtype=torch.float32, device="cuda")
    need = fp4.logits_topk_workspace_bytes("mxfp4", T, case.B, H, 1, 64, case.block_table.shape[1],
                                           oc, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        fp4.logits_topk_paged(q, qs, w, kf, ks, bt, cu, lens, fmt="mxfp4", out_cols=oc, k=k,
                              out_idx=idx, out_vals=vals, workspace=ws)

    g = _capture(call)
    for v, meta in enumerate(_logits_variants(case, np.random.default_rng(31 + T), 2)):
        bt.copy_(torch.from_numpy(meta["block_table"]))
        cu.copy_(torch.from_numpy(meta["cu_seqlens_q"]))
        lens.copy_(torch.from_numpy(meta["row_lens"]))
        torch.cuda.synchronize()
        c = _with(case, meta)
        ref, tb, inexact = orc.logits_paged(c.fmt, c.q_fp4, c.q_scale, c.w, c.k_fp4, c.k_scale,
                                            c.block_table, c.cu_seqlens_q, c.row_lens,
                                            c.page_size, oc, want_tolbase=True)
        assert inexact == 0
        e_out = fp4.logits_paged(q, qs, w, kf, ks, bt, cu, lens, fmt="mxfp4", out_cols=oc)
        e_idx, e_vals = fp4.topk(e_out, k, lens)
        torch.cuda.synchronize()
        e_idx, e_vals = e_idx.cpu().numpy(), e_vals.cpu().numpy()
        for rep in range(2):
            say(f"[gpu] graph replay: fused logits + top-{k}, T={T}, variant {v}, replay {rep}")
            idx.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            gi, gv = idx.cpu().numpy(), vals.cpu().numpy()
            np.testing.assert_array_equal(gi, e_idx)
            np.testing.assert_array_equal(gv.view(np.uint32), e_vals.view(np.uint32))
            nd = check_topk_against_oracle(ref, tb, gi, k, np.minimum(c.row_lens, oc))
            say(f"    ok (ties within tolerance against the oracle's logits: {nd})")
