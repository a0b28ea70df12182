"""GPU parity of fp4idx_logits_paged against the CPU oracle.

Bar (per the weighted-head-sum rule): the -inf pattern is identical and every visible
logit is within 1e-6 * sum_h |w_h ReLU(dot_h)| of the oracle's correctly rounded value.
Per-head dots, exposed through one-hot weights, are compared bit for bit.
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import DOT_BOUND, check_logits, dev, gpu_logits, oracle_logits, say

pytestmark = pytest.mark.gpu


def _parity(case, rows=None):
    got = gpu_logits(case)
    ref, tb, inexact = oracle_logits(case, rows=rows)
    assert inexact == 0
    worst = check_logits(got, ref, tb, rows=rows)
    say(f"    worst error / tolerance = {worst:.3f}")
    return got, ref


def test_config0_decode_ctx2048():
    _parity(wl.config0())


@pytest.mark.parametrize("ctx", [16384, 100_000])
def test_config1_decode_contexts(ctx):
    _parity(wl.config1(ctx))


def test_config1_400k_all_rows():
    _parity(wl.config1(400_000))


def test_config2_batched_decode_all_rows():
    _parity(wl.config2())


SMALL = [
    dict(name="ragged_multi_request", q_per_req=[1, 7, 0, 4], ctx=[70, 300, 5, 129], H=32),
    dict(name="heads_not_multiple_of_16", q_per_req=[3, 2], ctx=[200, 90], H=5),
    dict(name="gqa_two_key_heads", q_per_req=[4], ctx=[257], H=6, Hkv=2),
    dict(name="page128", q_per_req=[2, 2], ctx=[300, 129], H=16, page=128),
    dict(name="wide_scales", q_per_req=[4], ctx=[513], H=32, e8_lo=120, e8_hi=134),
    dict(name="single_row_requests", q_per_req=[1] * 9, ctx=[64 * i + 3 for i in range(9)], H=64),
    dict(name="h128", q_per_req=[2], ctx=[100], H=128),
    dict(name="nvfp4_decode", q_per_req=[4, 1], ctx=[333, 64], H=32, fmt=wl.NVFP4),
    dict(name="nvfp4_gqa", q_per_req=[2], ctx=[150], H=8, Hkv=4, fmt=wl.NVFP4),
    # many rows per request: workgroups of four row blocks, a partial last group and
    # row blocks that straddle two requests
    dict(name="prefill_rows_major", q_per_req=[71, 60], ctx=[700, 260], H=64),
    dict(name="prefill_rows_major_h32", q_per_req=[130], ctx=[1000], H=32),
    dict(name="prefill_rows_major_nvfp4", q_per_req=[9, 67], ctx=[90, 400], H=16, fmt=wl.NVFP4),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s["name"] for s in SMALL])
def test_small_shapes(spec):
    spec = dict(spec)
    name = spec.pop("name")
    case = wl.make_logits(name, seed=zlib.crc32(name.encode()) % 1000, **spec)
    # also exercise rows that see less than the whole context and out_cols past it
    case.row_lens = np.maximum(case.row_lens - np.arange(case.T, dtype=np.int32) % 3, 0)
    case.out_cols = int(max(spec["ctx"]) + 37)
    _parity(case)


def test_visibility_boundaries():
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256]
    case = wl.make_logits("bounds", q_per_req=[len(lens)], ctx=[256], H=32, seed=5,
                          row_lens=lens, out_cols=300)
    _parity(case)


def test_invalid_pages_and_rows_outside_requests():
    """A -1 page and a page past the cache are invisible; the last row lies past
    cu_seqlens_q[B], belongs to no request and must be -inf everywhere."""
    case = wl.make_logits("invalid", q_per_req=[3, 2], ctx=[300, 200], H=32, seed=8)
    case.block_table[0, 1] = -1
    case.block_table[1, 2] = case.num_pages + 5
    case.cu_seqlens_q[-1] = case.T - 1
    got, _ = _parity(case)
    assert np.all(got[case.T - 1] == -np.inf)
    assert np.all(np.isfinite(got[case.T - 2, :128]))


def test_page_permutation_gives_identical_logits():
    case = wl.make_logits("perm", q_per_req=[4], ctx=[1000], H=32, seed=12)
    a = gpu_logits(case)
    rng = np.random.default_rng(3)
    newpos = rng.permutation(case.num_pages)
    k2 = np.empty_like(case.k_fp4)
    s2 = np.empty_like(case.k_scale)
    k2[newpos] = case.k_fp4
    s2[newpos] = case.k_scale
    bt = case.block_table.copy()
    bt[bt >= 0] = newpos[bt[bt >= 0]]
    case.k_fp4, case.k_scale, case.block_table = k2, s2, bt
    b = gpu_logits(case)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_nonfinite_queries_leave_invisible_positions_neg_inf():
    case = wl.make_logits("nanq", q_per_req=[4], ctx=[500], H=32, seed=9, fmt=wl.NVFP4,
                          row_lens=[500, 100, 0, 1], out_cols=520)
    case.q_scale[1, 3, 2] = 0x7F   # NaN scale
    case.q_scale[2, :, :] = 0xFF   # NaN everywhere in a row that sees nothing
    got = gpu_logits(case)
    assert np.all(got[1, 100:] == -np.inf)
    assert np.all(got[2, :] == -np.inf)
    assert np.all(got[3, 1:] == -np.inf)
    assert np.all(np.isfinite(got[0, :500])) and np.all(got[0, 500:] == -np.inf)
    # visible positions too: a NaN head dot counts as 0 in fmax(x, 0) on both sides
    ref, tb, _ = oracle_logits(case)
    check_logits(got, ref, tb)


def test_noncontiguous_query_rows_and_combined_pages():
    """q/w rows with padding between them; keys in the combined page form (nibbles
    then scales inside one buffer per page)."""
    case = wl.make_logits("strided", q_per_req=[4], ctx=[700], H=32, seed=14)
    ref, tb, _ = oracle_logits(case)
    T, H = case.T, case.H
    qbig = np.zeros((T, H + 3, 64), np.uint8)
    qbig[:, :H] = case.q_fp4
    sbig = np.zeros((T, H + 1, 4), np.uint8)
    sbig[:, :H] = case.q_scale
    wbig = np.zeros((T, H + 7), np.float32)
    wbig[:, :H] = case.w
    P, page = case.num_pages, case.page_size
    comb = np.zeros((P, page * 68), np.uint8)
    comb[:, :page * 64] = case.k_fp4.reshape(P, page * 64)
    comb[:, page * 64:] = case.k_scale.reshape(P, page * 4)
    q_t = dev(qbig)[:, :H]
    s_t = dev(sbig)[:, :H]
    w_t = dev(wbig)[:, :H]
    comb_t = dev(comb)
    k_view = comb_t[:, :page * 64].view(P, 1, page, 64)
    ks_view = comb_t[:, page * 64:].view(P, 1, page, 4)
    say("[gpu] logits strided rows + combined pages")
    out = fp4.logits_paged(q_t, s_t, w_t, k_view, ks_view, dev(case.block_table),
                           dev(case.cu_seqlens_q), dev(case.row_lens), fmt=0,
                           out_cols=case.out_cols)
    torch.cuda.synchronize()
    check_logits(out.cpu().numpy(), ref, tb)


def _flip_sign(packed):
    return packed ^ np.uint8(0x88)


def _one_hot_head_dots(fmt, heads, **kw):
    """Per-head dots through one-hot head weights: w = e_h gives ReLU(dot_h) with no
    further rounding; flipping every query sign bit gives ReLU(-dot_h).  Returns (bit-exact
    count, total) over the visible values; every dot is held to DOT_BOUND[fmt] *
    sum_d |q_d k_d| and to the oracle's -inf pattern."""
    base = wl.make_logits("onehot", fmt=fmt, **kw)
    Hkv = base.Hkv
    R = base.H // Hkv
    mism = total = 0
    for h in heads:
        hk = h // R
        K = orc.dequant(fmt, base.k_fp4[:, hk], base.k_scale[:, hk])   # [P, page, 128]
        n_keys = int(base.row_lens.max())
        npg = -(-n_keys // base.page_size)
        Kl = K[base.block_table[0, :npg]].reshape(-1, 128)[:n_keys]     # logical order
        for sign in (1, -1):
            c = wl.make_logits("onehot", fmt=fmt, **kw)
            c.w[:] = 0
            c.w[:, h] = 1.0
            if sign < 0:
                c.q_fp4 = _flip_sign(c.q_fp4)
            got = gpu_logits(c)
            ref, _, inexact = oracle_logits(c)
            assert inexact == 0
            Q = orc.dequant(fmt, c.q_fp4[:, h], c.q_scale[:, h])
            absbase = np.abs(Q) @ np.abs(Kl).T
            vis = ref != -np.inf
            assert np.array_equal(got == -np.inf, ~vis)
            mism += int((got[vis] != ref[vis]).sum())
            total += int(vis.sum())
            err = np.abs(got[vis].astype(np.float64) - ref[vis])
            assert np.all(err <= DOT_BOUND[fmt] * absbase[:, :ref.shape[1]][vis])
    return total - mism, total


def test_per_head_dots_bit_exact_at_scale_codes_123_131():
    """MXFP4: the scaled MFMA forms each 32-element block sum exactly, scales it and adds
    the four block values in fp32; at scale codes 123..131 (configs 0, 1 and 4) every one
    of these per-head dots is the correctly rounded value."""
    ok, total = _one_hot_head_dots(wl.MXFP4, (0, 5, 17, 31), q_per_req=[4], ctx=[640], H=32,
                                   seed=31, e8_lo=123, e8_hi=131)
    say(f"    per-head bit-exact: {ok}/{total}")
    assert ok == total


def test_per_head_dots_at_scale_codes_120_134():
    """Config 2's wider code range: a block addition can round; the exact fraction is
    reported and held to the 2^-22 bound everywhere (measured 98.8%)."""
    ok, total = _one_hot_head_dots(wl.MXFP4, (0, 5, 17, 31), q_per_req=[4], ctx=[640], H=32,
                                   seed=31, e8_lo=120, e8_hi=134)
    say(f"    per-head bit-exact: {ok}/{total} = {ok / total:.4f}")
    assert ok >= 0.98 * total


def test_per_head_dots_nvfp4():
    """NVFP4 (config 3's E4M3 codes): four fp16 MFMAs of 32 exact products, accumulated in
    fp32; the bit-exact fraction is reported and asserted (measured 95.0%), every dot is
    within the NVFP4 bound."""
    ok, total = _one_hot_head_dots(wl.NVFP4, (0, 3, 6), q_per_req=[4], ctx=[700], H=8, Hkv=2,
                                   seed=37)
    say(f"    per-head bit-exact: {ok}/{total} = {ok / total:.4f}")
    assert ok >= 0.94 * total


# ---- long causal prefill at full size: 32768 x 32768 logits stay on the device; the
# oracle checks 256 seeded sampled rows plus the boundary rows, in two halves
_C4_FORCED = [0, 2046, 2047, 2048, 32767]


@pytest.fixture(scope="module")
def config4_gpu():
    case = wl.config4()
    rng = np.random.default_rng(1040)
    sampled = rng.choice(case.T, 256, replace=False)
    halves = [np.unique(np.concatenate([sampled[:128], _C4_FORCED])), np.unique(sampled[128:])]
    rows = np.unique(np.concatenate(halves))
    say(f"[gpu] logits {case.name} T={case.T} H={case.H} out_cols={case.out_cols} (+ top-2048)")
    out = fp4.logits_paged(dev(case.q_fp4), dev(case.q_scale), dev(case.w), dev(case.k_fp4),
                           dev(case.k_scale), dev(case.block_table), dev(case.cu_seqlens_q),
                           dev(case.row_lens), fmt=case.fmt, out_cols=case.out_cols)
    idx, _ = fp4.topk(out, 2048, dev(case.row_lens))
    torch.cuda.synchronize()
    sel = torch.from_numpy(rows).to(out.device)
    got = dict(zip(rows.tolist(), out.index_select(0, sel).cpu().numpy()))
    gidx = dict(zip(rows.tolist(), idx.index_select(0, sel).cpu().numpy()))
    del out, idx
    torch.cuda.empty_cache()
    return case, halves, got, gidx


@pytest.mark.parametrize("half", [0, 1])
def test_config4_prefill_sampled_rows_and_topk(config4_gpu, half):
    case, halves, got, gidx = config4_gpu
    rows = halves[half]
    ref, tb, inexact = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                        case.k_scale, case.block_table, case.cu_seqlens_q,
                                        case.row_lens, case.page_size, case.out_cols,
                                        rows=rows, want_tolbase=True, compact=True)
    assert inexact == 0
    g = np.stack([got[t] for t in rows.tolist()])
    worst = check_logits(g, ref, tb)
    say(f"    {rows.size} rows, worst error / tolerance = {worst:.3f}")
    lens = case.row_lens[rows]
    oi, _ = orc.topk(ref, 2048, lens)
    ndiff = 0
    for i, t in enumerate(rows.tolist()):
        a, b = set(gidx[t][gidx[t] >= 0].tolist()), set(oi[i][oi[i] >= 0].tolist())
        assert len(a) == len(b) == min(2048, int(lens[i]))
        assert np.all(gidx[t][len(a):] == -1)
        sel = np.array(sorted(b))
        kcol = sel[np.argmin(ref[i][sel])]             # the oracle's k-th largest
        for c in a ^ b:
            gap = abs(float(ref[i, c]) - float(ref[i, kcol]))
            assert gap <= 1e-6 * (float(tb[i, c]) + float(tb[i, kcol])) + 1e-30, (t, c)
        ndiff += len(a ^ b)
    say(f"    top-2048 symmetric differences (ties within tolerance): {ndiff}")
