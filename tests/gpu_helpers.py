"""Helpers shared by the GPU parity tests: upload a workload case, run the HIP library
through its Python binding, run the oracle on the same host arrays, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc


# Per-head dot bound, |gpu - exact| <= DOT_BOUND[fmt] * sum_d |q_d k_d|:
#  MXFP4: the scaled FP4 matrix core forms each 32-element block sum exactly, scales it
#         and adds the four block values to the fp32 accumulator in order (measured: every
#         dot bit-exact at scale codes 123..131), so at most three roundings: 2^-22.
#  NVFP4: four fp16 MFMAs of 32 exact products each, chained through the accumulator.
#         How one such instruction adds its products is not documented and no exact-sum
#         model reproduces it (measured: up to 4.6 * 2^-24 * (sum |products| + |C|) for a
#         single instruction); the bound assumes only one rounding per addition, in any
#         order, over the 128 products: 128 * 2^-24 = 2^-17.
DOT_BOUND = {0: 2.0 ** -22, 1: 2.0 ** -17}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def gpu_logits(case, out_cols=None):
    out_cols = case.out_cols if out_cols is None else out_cols
    say(f"[gpu] logits {case.name} T={case.T} H={case.H} Hkv={case.Hkv} B={case.B} "
        f"page={case.page_size} out_cols={out_cols} fmt={case.fmt}")
    out = fp4.logits_paged(dev(case.q_fp4), dev(case.q_scale), dev(case.w), dev(case.k_fp4),
                           dev(case.k_scale), dev(case.block_table), dev(case.cu_seqlens_q),
                           dev(case.row_lens), fmt=case.fmt, out_cols=out_cols)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_logits(case, rows=None, out_cols=None):
    out_cols = case.out_cols if out_cols is None else out_cols
    return orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4, case.k_scale,
                            case.block_table, case.cu_seqlens_q, case.row_lens, case.page_size,
                            out_cols, rows=rows, want_tolbase=True)


def check_logits(got, ref, tolbase, rows=None, rel=1e-6):
    """Parity rule for the weighted head sums: identical -inf pattern; elsewhere
    |got - ref| <= rel * sum_h |w_h ReLU(dot_h)| (and +-0 when that sum is 0)."""
    rows = range(got.shape[0]) if rows is None else rows
    worst = 0.0
    for t in rows:
        g, r, tb = got[t], ref[t], tolbase[t]
        inv = r == -np.inf
        assert np.array_equal(g == -np.inf, inv), f"row {t}: -inf pattern differs"
        vis = ~inv
        err = np.abs(g[vis].astype(np.float64) - r[vis].astype(np.float64))
        lim = rel * tb[vis].astype(np.float64)
        bad = err > lim
        assert not bad.any(), (f"row {t}: {bad.sum()} values outside tolerance, e.g. col "
                               f"{np.nonzero(vis)[0][np.argmax(bad)]} got {g[vis][bad][0]!r} "
                               f"ref {r[vis][bad][0]!r} base {tb[vis][bad][0]!r}")
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(lim > 0, err / np.where(lim > 0, lim, 1), 0)
        if q.size:
            worst = max(worst, float(q.max()))
    return worst


def gpu_block_scores(case):
    say(f"[gpu] block_scores {case.name} Tq={case.Tq} Hq={case.Hq} Hkv={case.Hkv} B={case.B} "
        f"fmt={case.fmt} causal={case.causal} qo={'yes' if case.qo_offset is not None else 'no'}")
    out = fp4.block_scores(dev(case.q_fp4), dev(case.k_fp4), dev(case.q_scale), dev(case.k_scale),
                           dev(case.cu_seqlens_q), dev(case.cu_seqlens_k), dev(case.cu_page_offsets),
                           max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k,
                           kv_indices=dev(case.kv_indices), fmt=case.fmt, causal=case.causal,
                           qo_offset=None if case.qo_offset is None else dev(case.qo_offset))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_block_scores(case, rows=None):
    return orc.block_scores(case.fmt, case.q_fp4, case.q_scale, case.k_fp4, case.k_scale,
                            case.cu_seqlens_q, case.cu_seqlens_k, case.cu_page_offsets,
                            case.kv_indices, case.qo_offset, case.max_seqlen_k, case.causal,
                            rows=rows, want_errbase=True)


def gpu_topk(scores_np, k, row_lens=None):
    s = dev(scores_np.astype(np.float32))
    rl = None if row_lens is None else dev(np.asarray(row_lens, np.int32))
    say(f"[gpu] topk rows={s.shape[0]} cols={s.shape[1]} k={k}")
    idx, vals = fp4.topk(s, k, rl)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


def check_topk_against_oracle(ref, tb, gidx, k, lens, label="rows"):
    """Tie-tolerant comparison of GPU top-k indices with the oracle's top-k of its own
    scores `ref` (rows of the same length as gidx): the chosen sets have the oracle's
    size, are listed in increasing column order and -1 padded, and may differ only in
    columns whose oracle score ties with the oracle's k-th within the logits tolerance
    (1e-6 of the summed |w ReLU(dot)| of both columns).  Returns the number of such
    columns."""
    oi, _ = orc.topk(ref, k, lens)
    ndiff = 0
    for i in range(ref.shape[0]):
        g = gidx[i]
        a, b = set(g[g >= 0].tolist()), set(oi[i][oi[i] >= 0].tolist())
        assert len(a) == len(b), (label, i, len(a), len(b))
        assert np.all(g[len(a):] == -1) and np.all(np.diff(g[:len(a)]) > 0)
        if not b:
            continue
        sel = np.array(sorted(b))
        kcol = sel[np.argmin(ref[i][sel])]
        for c in a ^ b:
            gap = abs(float(ref[i, c]) - float(ref[i, kcol]))
            assert gap <= 1e-6 * (float(tb[i, c]) + float(tb[i, kcol])) + 1e-30, (label, i, c)
        ndiff += len(a ^ b)
    return ndiff
