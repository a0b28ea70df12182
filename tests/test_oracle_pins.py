"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins and where the fact comes from: a value printed on the
pages (fixtures under tests/golden/), a library routine (torch's float8 dtypes, numpy's
float64 matmul and sort), a closed form, or an invariant of the definition.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


# ---------------------------------------------------------------- library / closed-form decoders
def e2m1_bitfield(n):
    """OCP E2M1 read as a float format: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    s, e, m = (n >> 3) & 1, (n >> 1) & 3, n & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def torch_e8m0(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def lib_dequant(fmt, packed, scales):
    """Dequantize with library decoders only (torch float8 views + the OCP bit-field
    E2M1); shares nothing with the oracle's decode."""
    packed = np.asarray(packed, np.uint8)
    lo = packed & 15
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], 128)
    lut = np.array([e2m1_bitfield(n) for n in range(16)])
    vals = lut[nib]
    S = 32 if fmt == wl.MXFP4 else 16
    sc = torch_e8m0(scales) if fmt == wl.MXFP4 else torch_e4m3(scales)
    return vals * np.repeat(sc, S, axis=-1)


# ---------------------------------------------------------------- decode pins
def test_e2m1_matches_issue_level_table_and_not_the_buggy_decode():
    for idx, val, bug in _rows("e2m1_levels.txt"):
        i = int(idx)
        assert orc.e2m1(i) == float(val)
        assert orc.e2m1(i | 8) == -float(val)
        if float(val) != float(bug):
            assert orc.e2m1(i) != float(bug)


def test_e2m1_matches_ocp_bitfield_form_for_all_16_codes():
    for n in range(16):
        a, b = orc.e2m1(n), e2m1_bitfield(n)
        assert a == b and math.copysign(1, a) == math.copysign(1, b), n


def test_e8m0_matches_torch_for_codes_0_to_254_and_literal_formula_at_255():
    t = torch_e8m0(np.arange(256))
    for c in range(255):
        assert orc.e8m0(c) == t[c], c
    # torch reads 255 as NaN; the literal 2^(c-127) is 2^128 (finite in double, inf once
    # rounded to fp32).  The stored codes are 1..254, so parity is required only there.
    assert math.isnan(t[255])
    assert orc.e8m0(255) == 2.0 ** 128
    assert np.float32(orc.e8m0(255)) == np.float32(np.inf)


def test_e4m3_matches_torch_for_all_256_codes():
    t = torch_e4m3(np.arange(256))
    for c in range(256):
        a = orc.e4m3(c)
        if math.isnan(t[c]):
            assert math.isnan(a), c
        else:
            assert a == t[c] and math.copysign(1, a) == math.copysign(1, t[c]), c


def test_nibble_order_matches_issue_fixture():
    for byte, v0, v1 in _rows("nibble_order.txt"):
        packed = np.zeros(64, np.uint8)
        packed[5] = int(byte, 16)
        vals = orc.dequant(wl.MXFP4, packed, np.full(4, 127, np.uint8))
        assert vals[10] == float(v0) and math.copysign(1, vals[10]) == math.copysign(1, float(v0))
        assert vals[11] == float(v1) and math.copysign(1, vals[11]) == math.copysign(1, float(v1))


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4])
def test_dequant_matches_library_decoders(fmt):
    rng = np.random.default_rng(7)
    G = wl.groups(fmt)
    packed = rng.integers(0, 256, (50, 64), dtype=np.uint8)
    if fmt == wl.MXFP4:
        scales = rng.integers(100, 160, (50, G), dtype=np.uint8)
    else:
        scales = rng.integers(0, 256, (50, G), dtype=np.uint8)
        scales[(scales & 0x7F) == 0x7F] = 0x38
    np.testing.assert_array_equal(orc.dequant(fmt, packed, scales), lib_dequant(fmt, packed, scales))


# ---------------------------------------------------------------- dot pins
def test_dot_closed_forms():
    ones = np.full(64, 0x22, np.uint8)  # every element code 2 = 1.0
    unit = np.full(4, 127, np.uint8)
    q = orc.dequant(wl.MXFP4, ones, unit)
    v, exact, a = orc.dot(q, q)
    assert (v, exact, a) == (128.0, True, 128.0)
    sixes = np.full(64, 0x77, np.uint8)  # code 7 = 6.0
    for sa, sb in [(127, 127), (130, 120), (100, 150)]:
        q = orc.dequant(wl.MXFP4, sixes, np.full(4, sa, np.uint8))
        k = orc.dequant(wl.MXFP4, sixes, np.full(4, sb, np.uint8))
        v, exact, _ = orc.dot(q, k)
        assert exact and v == 4 * 36 * 32 * 2.0 ** (sa - 127 + sb - 127)
    # one-hot: a single product survives
    a = np.zeros(64, np.uint8)
    b = np.zeros(64, np.uint8)
    a[17] = 0x50  # element 35 = code 5 = 3.0
    b[17] = 0xF0  # element 35 = code 15 = -6.0
    b[3] = 0x77   # elements 6,7 -- multiplied by zeros
    q = orc.dequant(wl.MXFP4, a, np.array([127, 129, 127, 127], np.uint8))
    k = orc.dequant(wl.MXFP4, b, np.array([127, 126, 127, 127], np.uint8))
    assert orc.dot(q, k)[0] == 3.0 * 4 * -6.0 * 0.5


@pytest.mark.parametrize("fmt,lo,hi", [(wl.MXFP4, 123, 131), (wl.MXFP4, 120, 134), (wl.NVFP4, 0, 0)])
def test_dot_matches_numpy_float64_matmul_and_is_exact_on_workload_distributions(fmt, lo, hi):
    rng = np.random.default_rng(11)
    G = wl.groups(fmt)
    n = 300
    pq = rng.integers(0, 256, (n, 64), dtype=np.uint8)
    pk = rng.integers(0, 256, (n, 64), dtype=np.uint8)
    if fmt == wl.MXFP4:
        sq = rng.integers(lo, hi + 1, (n, G), dtype=np.uint8)
        sk = rng.integers(lo, hi + 1, (n, G), dtype=np.uint8)
    else:
        e = rng.integers(-4, 5, (2, n, G))
        m = rng.integers(0, 8, (2, n, G))
        c = (((e + 7) << 3) | m).astype(np.uint8)
        sq, sk = c[0], c[1]
    Q = lib_dequant(fmt, pq, sq)
    K = lib_dequant(fmt, pk, sk)
    ref = np.einsum("nd,nd->n", Q, K)  # float64; exact on these dyadic inputs (< 53 bits)
    qo = orc.dequant(fmt, pq, sq)
    ko = orc.dequant(fmt, pk, sk)
    for i in range(n):
        v, exact, _ = orc.dot(qo[i], ko[i])
        assert exact
        assert v == ref[i]


def test_dot_exactness_flag_turns_off_for_extreme_scale_spreads():
    q = np.zeros(128)
    k = np.zeros(128)
    q[0], k[0] = 2.0 ** 60, 1.0
    q[1], k[1] = 2.0 ** -60, 1.0
    v, exact, _ = orc.dot(q, k)
    assert not exact and v == 2.0 ** 60


# ---------------------------------------------------------------- logits pins
def _small_logits(seed=3, H=4, Hkv=1, ctx=(150, 70), q_per_req=(2, 3), fmt=wl.MXFP4, page=64):
    return wl.make_logits("small", fmt=fmt, q_per_req=list(q_per_req), ctx=list(ctx), H=H,
                          Hkv=Hkv, page=page, seed=seed)


def _run(case, **kw):
    return orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4, case.k_scale,
                            case.block_table, case.cu_seqlens_q, case.row_lens, case.page_size,
                            case.out_cols, **kw)


def _logical_keys(case, b, n):
    """Logical keys 0..n-1 of request b, found by scanning every physical page for the
    block-table entry that names it (no division / modulo arithmetic)."""
    Hkv, page = case.Hkv, case.page_size
    kp = np.zeros((n, Hkv, 64), np.uint8)
    ks = np.zeros((n, Hkv, case.k_scale.shape[-1]), np.uint8)
    pos = 0
    for lp in range(case.block_table.shape[1]):
        phys = case.block_table[b, lp]
        for off in range(page):
            if pos >= n:
                return kp, ks
            kp[pos] = case.k_fp4[phys, :, off]
            ks[pos] = case.k_scale[phys, :, off]
            pos += 1
    return kp, ks


@pytest.mark.parametrize("H,Hkv,fmt", [(4, 1, wl.MXFP4), (6, 2, wl.MXFP4), (4, 2, wl.NVFP4)])
def test_one_hot_weights_expose_relu_of_each_head_dot(H, Hkv, fmt):
    case = _small_logits(H=H, Hkv=Hkv, fmt=fmt)
    R = H // Hkv
    for h in range(H):
        case.w[:] = 0
        case.w[:, h] = 1.0
        out, _, inexact = _run(case)
        assert inexact == 0
        for b in range(case.B):
            rows = range(case.cu_seqlens_q[b], case.cu_seqlens_q[b + 1])
            n = int(case.row_lens[list(rows)].max())
            kp, ks = _logical_keys(case, b, n)
            K = lib_dequant(fmt, kp[:, h // R], ks[:, h // R])
            for t in rows:
                q = lib_dequant(fmt, case.q_fp4[t, h], case.q_scale[t, h])
                want = np.maximum(K @ q, 0).astype(np.float32)
                got = out[t, :n]
                np.testing.assert_array_equal(got, want)


def test_head_sum_is_linear_in_weights_within_tolerance():
    case = _small_logits(H=5, seed=9)
    out, tb, _ = _run(case, want_tolbase=True)
    w = case.w.copy()
    parts = []
    for h in range(case.H):
        case.w[:] = 0
        case.w[:, h] = 1.0
        parts.append(_run(case)[0].astype(np.float64))
    vis = np.isfinite(out)
    comb = sum(w[:, h:h + 1].astype(np.float64) * np.where(vis, parts[h], 0) for h in range(case.H))
    assert np.all(np.abs(out[vis] - comb[vis]) <= 1e-6 * tb[vis] + 1e-30)


def test_visibility_counts_and_boundaries():
    case = wl.make_logits("bounds", q_per_req=[12], ctx=[200], H=2, seed=4,
                          row_lens=[0, 1, 63, 64, 65, 127, 128, 129, 191, 192, 199, 200],
                          out_cols=256)
    out, _, _ = _run(case)
    for t in range(case.T):
        L = case.row_lens[t]
        assert np.all(np.isfinite(out[t, :L]))
        assert np.all(out[t, L:] == -np.inf)


def test_page_permutation_does_not_change_logits():
    case = _small_logits(seed=21, ctx=(300, 130))
    out1, _, _ = _run(case)
    # move every physical page to a new slot and rewrite the table to match
    rng = np.random.default_rng(5)
    P = case.num_pages
    newpos = rng.permutation(P)
    k2 = np.empty_like(case.k_fp4)
    s2 = np.empty_like(case.k_scale)
    k2[newpos] = case.k_fp4
    s2[newpos] = case.k_scale
    bt = case.block_table.copy()
    bt[bt >= 0] = newpos[bt[bt >= 0]]
    case.k_fp4, case.k_scale, case.block_table = k2, s2, bt
    out2, _, _ = _run(case)
    np.testing.assert_array_equal(out1, out2)


def test_invisible_positions_stay_neg_inf_with_nan_queries():
    case = _small_logits(seed=5, fmt=wl.NVFP4, ctx=(100, 40), q_per_req=(1, 1))
    ref, _, _ = _run(case)
    case.q_scale[0, 1, 3] = 0x7F  # NaN scale for one head of row 0
    out, _, _ = _run(case)
    assert np.all(out[0, 100:] == -np.inf)
    assert np.all(np.isfinite(out[1, :40])) and np.all(out[1, 40:] == -np.inf)
    # ReLU is fmax(x, 0): the NaN head adds 0, so row 0 equals the same row with head 1's
    # weight set to 0 (dot products are exact, so this holds to the last bit)
    case.q_scale[0, 1, 3] = case.q_scale[0, 1, 2]
    case.w[0, 1] = 0.0
    zeroed, _, _ = _run(case)
    np.testing.assert_array_equal(out[0], zeroed[0])
    assert not np.array_equal(out[0, :100], ref[0, :100])


def test_invalid_page_ids_are_invisible():
    case = _small_logits(seed=6, ctx=(200, 70))
    case.block_table[0, 1] = -1
    case.block_table[1, 0] = case.num_pages + 3
    out, _, _ = _run(case)
    r0 = range(case.cu_seqlens_q[0], case.cu_seqlens_q[1])
    for t in r0:
        assert np.all(out[t, 64:128] == -np.inf)
        assert np.all(np.isfinite(out[t, :64])) and np.all(np.isfinite(out[t, 128:200]))
    for t in range(case.cu_seqlens_q[1], case.cu_seqlens_q[2]):
        assert np.all(out[t, :64] == -np.inf)


# ---------------------------------------------------------------- block-score pins
def test_rows_outside_every_request_see_nothing():
    """A row t >= cu_seqlens_q[B] belongs to no request, so it sees no key and is -inf
    everywhere (with tolerance base 0), however long its row_lens entry.  Pinned against
    the same rows counted into the last request, where they see that request's keys
    (finite values): an oracle that gave an orphan row to request B-1 fails here.  The
    rows inside requests must not change."""
    case = _small_logits(seed=17, ctx=(150, 90), q_per_req=(2, 3))
    full, _, _ = _run(case)
    T = case.T
    last = range(int(case.cu_seqlens_q[1]), T)
    for t in last:
        assert np.all(np.isfinite(full[t, :90])) and np.all(full[t, 90:] == -np.inf)
    case.cu_seqlens_q[-1] = T - 2            # the last two rows now belong to no request
    cut, tb, _ = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                  case.k_scale, case.block_table, case.cu_seqlens_q,
                                  case.row_lens, case.page_size, case.out_cols,
                                  want_tolbase=True)
    assert np.all(cut[T - 2:] == -np.inf) and np.all(tb[T - 2:] == 0)
    np.testing.assert_array_equal(cut[:T - 2], full[:T - 2])


def test_causal_visibility_fixture():
    for q_len, k_len, qo, ql, vis in _rows("causal_visibility.txt"):
        q_len, k_len, ql = int(q_len), int(k_len), int(ql)
        want = [] if vis == "none" else [int(x) for x in vis.split(",")]
        # a key is seen iff its one-hot score block reports it: give key j a value that
        # identifies it (dot = j+1 for the single query that is probed)
        case = wl.make_block("fx", fmt=wl.MXFP4, q_lens=[q_len], k_lens=[k_len], Hq=1, Hkv=1,
                             seed=1, qo_offset=None if qo == "-" else [int(qo)])
        case.q_fp4[:] = 0
        case.q_scale[:] = 127
        case.q_fp4[:, 0, 0] = 0x02  # q[0] = 1.0, rest 0
        case.k_fp4[:] = 0
        case.k_scale[:] = 127
        seen = []
        for j in range(k_len):
            # key j alone carries a positive value; all other keys score 0
            case.k_fp4[:] = 0
            phys = case.kv_indices[j // 128]
            case.k_fp4[phys, 0, j % 128, 0] = 0x02
            out, _, _ = orc.block_scores(case.fmt, case.q_fp4, case.q_scale, case.k_fp4,
                                         case.k_scale, case.cu_seqlens_q, case.cu_seqlens_k,
                                         case.cu_page_offsets, case.kv_indices, case.qo_offset,
                                         case.max_seqlen_k, True)
            if out[0, 0, ql] == 1.0:
                seen.append(j)
        assert seen == want, (q_len, k_len, qo, ql)


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4])
@pytest.mark.parametrize("causal", [True, False])
def test_block_scores_brute_force_against_library_dot(fmt, causal):
    case = wl.make_block("bf", fmt=fmt, q_lens=[5, 3], k_lens=[300, 129], Hq=4, Hkv=2, seed=13,
                         causal=causal)
    out, _, inexact = orc.block_scores(case.fmt, case.q_fp4, case.q_scale, case.k_fp4,
                                       case.k_scale, case.cu_seqlens_q, case.cu_seqlens_k,
                                       case.cu_page_offsets, case.kv_indices, None,
                                       case.max_seqlen_k, causal)
    assert inexact == 0
    R = case.Hq // case.Hkv
    for b in range(case.B):
        ql = case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b]
        kl = case.cu_seqlens_k[b + 1] - case.cu_seqlens_k[b]
        pages = case.kv_indices[case.cu_page_offsets[b]:case.cu_page_offsets[b + 1]]
        for hq in range(case.Hq):
            K = np.concatenate([lib_dequant(fmt, case.k_fp4[p, hq // R], case.k_scale[p, hq // R])
                                for p in pages])[:kl]
            for qi in range(ql):
                qg = case.cu_seqlens_q[b] + qi
                s = K @ lib_dequant(fmt, case.q_fp4[qg, hq], case.q_scale[qg, hq])
                lim = kl if not causal else min(kl, qi + (kl - ql) + 1)
                for kb in range(case.ktiles):
                    seg = s[128 * kb:min(128 * kb + 128, lim)]
                    want = np.float32(seg.max()) if seg.size else -np.inf
                    assert out[hq, kb, qg] == want


def test_block_max_skips_nan_dots():
    """A NaN E4M3 code (0x7F) on one key makes that key's dots NaN; the block max is C's
    fmax, so it equals numpy's nanmax over the library-decoded dots of the block, and a
    query head whose dots are all NaN gets -inf blocks."""
    case = wl.make_block("nan", fmt=wl.NVFP4, q_lens=[4], k_lens=[200], Hq=2, Hkv=1, seed=19,
                         causal=False)
    p0 = int(case.kv_indices[0])
    case.k_scale[p0, 0, 7, 1] = 0x7F                 # key 7: NaN for every query
    case.q_scale[3, 1, 0] = 0xFF                     # query 3, head 1: every dot NaN
    out, _, _ = orc.block_scores(case.fmt, case.q_fp4, case.q_scale, case.k_fp4, case.k_scale,
                                 case.cu_seqlens_q, case.cu_seqlens_k, case.cu_page_offsets,
                                 case.kv_indices, None, case.max_seqlen_k, False)
    K = np.concatenate([lib_dequant(wl.NVFP4, case.k_fp4[p, 0], case.k_scale[p, 0])
                        for p in case.kv_indices])[:200]
    for hq in range(2):
        for q in range(4):
            with np.errstate(invalid="ignore"):
                s = K @ lib_dequant(wl.NVFP4, case.q_fp4[q, hq], case.q_scale[q, hq])
            for kb in range(2):
                seg = s[128 * kb:min(128 * kb + 128, 200)]
                want = -np.inf if np.all(np.isnan(seg)) else np.float32(np.nanmax(seg))
                assert out[hq, kb, q] == want, (hq, q, kb)
    assert np.all(out[1, :, 3] == -np.inf)


def test_block_max_equals_max_of_one_head_logits():
    """Cross-API: H=Hkv=1, w=1 logits on 128-token pages equal max(block score, 0)."""
    bc = wl.make_block("x", fmt=wl.MXFP4, q_lens=[2], k_lens=[300], Hq=1, Hkv=1, seed=17,
                       causal=False)
    out_b, _, _ = orc.block_scores(bc.fmt, bc.q_fp4, bc.q_scale, bc.k_fp4, bc.k_scale,
                                   bc.cu_seqlens_q, bc.cu_seqlens_k, bc.cu_page_offsets,
                                   bc.kv_indices, None, bc.max_seqlen_k, False)
    bt = np.full((1, 3), -1, np.int32)
    bt[0, :3] = bc.kv_indices
    lg, _, _ = orc.logits_paged(bc.fmt, bc.q_fp4, bc.q_scale, np.ones((2, 1), np.float32),
                                bc.k_fp4, bc.k_scale, bt, np.array([0, 2], np.int32),
                                np.array([300, 300], np.int32), 128, 300)
    for t in range(2):
        for kb in range(3):
            assert lg[t, 128 * kb:128 * kb + 128].max() == max(out_b[0, kb, t], 0.0)


# ---------------------------------------------------------------- top-k pins
def test_topk_matches_numpy_stable_sort():
    rng = np.random.default_rng(2)
    rows, cols, k = 6, 3000, 100
    s = rng.integers(-50, 50, (rows, cols)).astype(np.float32) / 4  # many ties
    s[0, :] = -np.inf
    s[1, 2000:] = -np.inf
    s[2, 5] = np.nan
    s[3, ::7] = -0.0
    lens = np.array([3000, 3000, 3000, 3000, 50, 0], np.int32)
    idx, vals = orc.topk(s, k, lens)
    for t in range(rows):
        L = min(lens[t], cols)
        v = s[t, :L].astype(np.float64)
        v = np.where(v == 0, 0.0, v)
        cand = np.nonzero(v > -np.inf)[0]
        order = cand[np.argsort(-v[cand], kind="stable")]
        want = np.sort(order[:k])
        m = len(want)
        np.testing.assert_array_equal(idx[t, :m], want)
        assert np.all(idx[t, m:] == -1)
        np.testing.assert_array_equal(vals[t, :m], s[t, want])
        assert np.all(vals[t, m:] == -np.inf)
        if m and m < len(cand):
            unsel = np.setdiff1d(cand, want)
            assert v[want].min() >= v[unsel].max()


def test_compact_rows_match_the_full_call():
    """The compact form of the logits call (only sampled rows, used where the full
    [T, out_cols] array would not fit) returns exactly the full call's rows."""
    case = wl.make_logits("compact", q_per_req=[3, 2, 4], ctx=[150, 90, 200], H=8, seed=12,
                          row_lens=[150, 149, 3, 90, 0, 200, 199, 64, 1], out_cols=210)
    rows = [7, 0, 4, 5, 2]
    full, _, _ = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                  case.k_scale, case.block_table, case.cu_seqlens_q, case.row_lens,
                                  case.page_size, case.out_cols)
    comp, _, _ = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                  case.k_scale, case.block_table, case.cu_seqlens_q, case.row_lens,
                                  case.page_size, case.out_cols, rows=rows, compact=True)
    np.testing.assert_array_equal(comp, full[sorted(rows)])


# ---------------------------------------------------------------- quantizer pins
def _golden_blocks():
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "quantize_blocks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "block":
                cur = dict(name=parts[1], code=int(parts[3]), x=np.zeros(32), nib=np.zeros(32, int))
                blocks.append(cur)
            else:
                i = int(parts[0])
                cur["x"][i] = float(parts[1])
                cur["nib"][i] = int(parts[2])
    return blocks


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b["name"])
def test_quantize_block_matches_hand_worked_fixture(blk):
    packed, code = orc.quantize_mx_block(blk["x"])
    assert code == blk["code"]
    nib = np.empty(32, int)
    nib[0::2] = packed & 15
    nib[1::2] = packed >> 4
    assert np.array_equal(nib, blk["nib"])


def _nearest_even_level(m):
    """numpy reference of the rounding rule: nearest of the eight magnitudes, ties to
    the even index."""
    lv = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(m[:, None] - lv[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = np.where(np.isclose(d, dmin, rtol=0, atol=0), np.arange(8)[None, :], 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=1)
    return np.where(even < 99, even, cand.min(axis=1))


def test_quantize_random_blocks_against_numpy_rounding_and_exponent_rule():
    rng = np.random.default_rng(21)
    for t in range(400):
        mag = 2.0 ** rng.integers(-20, 20)
        x = (rng.standard_normal(32) * mag).astype(np.float32).astype(np.float64)
        if t % 7 == 0:
            x[rng.integers(0, 32, 5)] = 0.0
        packed, code = orc.quantize_mx_block(x)
        amax = np.abs(x).max()
        assert code == int(np.clip(np.floor(np.log2(amax)) - 2 + 127, 1, 254))
        scale = 2.0 ** (code - 127)
        want = _nearest_even_level(np.abs(x) / scale)
        nib = np.empty(32, int)
        nib[0::2] = packed & 15
        nib[1::2] = packed >> 4
        assert np.array_equal(nib & 7, want)
        assert np.array_equal(nib >> 3, np.signbit(x).astype(int))
        # decoding with the library E2M1 / E8M0 decoders stays within half a grid step
        dec = lib_dequant(wl.MXFP4, np.concatenate([packed, np.zeros(48, np.uint8)]),
                          np.array([code, 127, 127, 127], np.uint8))[:32]
        step = np.where(np.abs(x) / scale >= 4, 2.0, np.where(np.abs(x) / scale >= 2, 1.0, 0.5))
        assert np.all(np.abs(dec - np.clip(x, -6 * scale, 6 * scale)) <= 0.5 * step * scale)


def test_quantize_store_scatters_by_slot():
    rng = np.random.default_rng(22)
    P, page = 5, 64
    kf = rng.integers(0, 256, (P, 1, page, 64), dtype=np.uint8)
    ks = rng.integers(0, 256, (P, 1, page, 4), dtype=np.uint8)
    keys = rng.standard_normal((7, 128))
    slots = np.array([3, 200, -1, 319, 64, 320, 0], np.int64)   # -1 and 320 are skipped
    of, os_ = orc.quantize_store(keys, slots, kf, ks)
    touched = np.zeros((P, page), bool)
    for n, s in enumerate(slots):
        if 0 <= s < P * page:
            pg, tok = divmod(int(s), page)
            touched[pg, tok] = True
            for g in range(4):
                pk, c = orc.quantize_mx_block(keys[n, 32 * g:32 * g + 32])
                assert np.array_equal(of[pg, 0, tok, 16 * g:16 * g + 16], pk)
                assert os_[pg, 0, tok, g] == c
    assert np.array_equal(of[:, 0][~touched], kf[:, 0][~touched])
    assert np.array_equal(os_[:, 0][~touched], ks[:, 0][~touched])


def test_block_topk_hand_worked():
    # Hq=1, Ktiles=5, Tq=2.  Query 0 sees blocks [3, 7, -inf, 7, 1]: top-2 = blocks 1 and
    # 3 (both 7; the tie keeps the smaller block first, and both fit); top-3 adds block 0.
    # Query 1 sees [nan, -inf, 2, -inf, -inf]: one finite block.
    s = np.array([[[3, np.nan], [7, -np.inf], [-np.inf, 2], [7, -np.inf], [1, -np.inf]]], np.float32)
    idx, cnt = orc.block_topk(s, 2)
    np.testing.assert_array_equal(idx[0], [[1, 3], [2, -1]])
    np.testing.assert_array_equal(cnt[0], [2, 1])
    idx, cnt = orc.block_topk(s, 3)
    np.testing.assert_array_equal(idx[0], [[0, 1, 3], [2, -1, -1]])
    np.testing.assert_array_equal(cnt[0], [3, 1])
    # a tie at the k-th place goes to the smaller block
    t = np.array([[[5], [4], [4], [4]]], np.float32)
    idx, cnt = orc.block_topk(t, 2)
    np.testing.assert_array_equal(idx[0, 0], [0, 1])


def test_block_topk_brute_force():
    rng = np.random.default_rng(9)
    Hq, Kt, Tq, k = 3, 40, 17, 6
    s = (rng.integers(-8, 8, (Hq, Kt, Tq)) / 2).astype(np.float32)
    s[rng.random(s.shape) < 0.3] = -np.inf
    s[0, :, 0] = -np.inf
    idx, cnt = orc.block_topk(s, k)
    for h in range(Hq):
        for q in range(Tq):
            col = s[h, :, q].astype(np.float64)
            fin = [b for b in range(Kt) if col[b] > -np.inf]
            best = sorted(fin, key=lambda b: (-col[b], b))[:k]
            want = sorted(best) + [-1] * (k - len(best))
            assert idx[h, q].tolist() == want
            assert cnt[h, q] == len(best)


# ---------------------------------------------------------------------------------------
# Sparse paged attention over the selected tokens (vLLM qsa_fp8 API page).
# ---------------------------------------------------------------------------------------

def test_qsa_offset_bits_is_the_least_width_that_holds_every_place():
    for page in range(1, 1025):
        b = orc.qsa_offset_bits(page)
        assert b >= 1 and (1 << b) >= page          # every place 0..page-1 fits in b bits
        assert b == 1 or (1 << (b - 1)) < page      # and b - 1 bits would not do


def _golden_slots():
    meta, table, rows = {}, [], []
    with open(os.path.join(GOLDEN, "qsa_slots.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "table":
                table.append([int(x) for x in rest.split()])
            elif key == "row":
                req, toks, want = rest.split("|")
                rows.append((int(req), [int(x) for x in toks.split()],
                             [int(x) for x in want.split()]))
            else:
                meta[key] = int(rest)
    return meta, np.array(table, np.int32), rows


def test_qsa_slots_match_hand_worked_fixture():
    meta, table, rows = _golden_slots()
    ind = np.array([r[1] for r in rows], np.int32)
    t2r = np.array([r[0] for r in rows], np.int32)
    assert ind.shape[1] == meta["topk"] + 1
    got = orc.qsa_slots(ind, table, t2r, meta["num_cache_blocks"], meta["page"],
                        meta["slot_cols"])
    np.testing.assert_array_equal(got, np.array([r[2] for r in rows], np.int32))


def _bf16_bits(x):
    return torch.as_tensor(x, dtype=torch.float64).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _qsa_case(rng, rows=3, Hq=8, Hkv=2, D=16, page=8, blocks=12, topk=10, combined=True):
    """Random small case: per-request block tables over a shuffled page pool, finite
    e4m3fn K/V codes (0x7F/0xFF excluded), bf16 q and gate."""
    codes = rng.integers(0, 256, size=(blocks, Hkv, page, 2 * D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                       # no NaN codes
    if combined:   # one cache [blocks, Hkv, page, 2D] seen as [blocks, page, Hkv, D] twice
        kv = codes.transpose(0, 2, 1, 3)
        k, v = kv[..., :D], kv[..., D:]
    else:          # separate caches; V's heads stored in reverse order (head stride -D)
        k = np.ascontiguousarray(codes[..., :D].transpose(0, 2, 1, 3))
        vbuf = np.ascontiguousarray(codes[..., D:].transpose(0, 2, 1, 3)[:, :, ::-1])
        v = vbuf[:, :, ::-1]
    width = blocks // rows
    perm = rng.permutation(blocks).astype(np.int32)
    table = perm[: rows * width].reshape(rows, width)
    ctx = width * page
    ind = np.full((rows, topk + 1), -1, np.int32)
    for r in range(rows):
        sel = np.sort(rng.choice(ctx, size=topk - 2, replace=False))
        ind[r, : topk - 2] = sel
        ind[r, topk] = topk - 2
    q = _bf16_bits(rng.standard_normal((rows, Hq, D)))
    gate = _bf16_bits(rng.standard_normal((rows, Hq, D)) * 2)
    t2r = np.arange(rows, dtype=np.int32)
    return dict(k=k, v=v, table=table, ind=ind, q=q, gate=gate, t2r=t2r, page=page,
                blocks=blocks, D=D, Hq=Hq, Hkv=Hkv)


def _qsa_run(c, softmax_scale=0.3, output_scale=1.0, slots=None, ind=None):
    ind = c["ind"] if ind is None else ind
    if slots is None:
        slots = orc.qsa_slots(ind, c["table"], c["t2r"], c["blocks"], c["page"])
    out, tb = orc.qsa_decode(c["q"], c["k"], c["v"], slots, ind,
                             orc.qsa_offset_bits(c["page"]), softmax_scale, output_scale,
                             c["gate"], want_tolbase=True)
    return out, tb


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def test_qsa_single_selected_token_outputs_its_value_row_gated():
    """One selected token takes all the probability: out = output_scale * V * sigmoid(gate)
    (V decoded by torch's float8_e4m3fn, not by the oracle's decoder)."""
    rng = np.random.default_rng(11)
    c = _qsa_case(rng)
    ind = c["ind"].copy()
    ind[:, 1:] = -1
    ind[:, -1] = 1
    out, _ = _qsa_run(c, output_scale=0.75, ind=ind)
    G = c["Hq"] // c["Hkv"]
    for r in range(ind.shape[0]):
        x = ind[r, 0]
        pg, place = c["table"][r, x // c["page"]], x % c["page"]
        for h in range(c["Hq"]):
            vrow = _e4m3_values(c["v"][pg, place, h // G])
            want = 0.75 * vrow * _sigmoid(_bf16_values(c["gate"][r, h]))
            np.testing.assert_allclose(out[r, h], want, rtol=1e-14, atol=0)


def test_qsa_equal_keys_average_the_values():
    """Every selected token of a row holds the same key: the weights are all 1/n and the
    output is the mean of the value rows."""
    rng = np.random.default_rng(12)
    c = _qsa_case(rng, combined=False)
    k = np.array(c["k"])          # writable copy, same strides as the separate V cache
    k[...] = k[0, 0, :, :][None, None]
    c["k"] = k
    out, _ = _qsa_run(c, softmax_scale=1.7)
    G = c["Hq"] // c["Hkv"]
    for r in range(c["ind"].shape[0]):
        n = c["ind"][r, -1]
        toks = c["ind"][r, :n]
        for h in range(c["Hq"]):
            vals = np.stack([_e4m3_values(c["v"][c["table"][r, x // c["page"]], x % c["page"],
                                                 h // G]) for x in toks])
            want = vals.mean(axis=0) * _sigmoid(_bf16_values(c["gate"][r, h]))
            np.testing.assert_allclose(out[r, h], want, rtol=1e-13, atol=1e-300)


def test_qsa_two_tokens_with_score_gap_ln3_weigh_three_to_one():
    """q = e_0, K_a[0] = 1, K_b[0] = 0 and softmax_scale = ln 3: scores ln 3 and 0, so the
    weights are 3/4 and 1/4; gate 0 halves the output."""
    D, page = 16, 4
    k = np.zeros((2, page, 1, D), np.uint8)
    v = np.zeros((2, page, 1, D), np.uint8)
    k[0, 1, 0, 0] = 0x38                                   # 1.0
    v[0, 1, 0, :] = 0x40                                   # 2.0
    v[1, 2, 0, :] = 0x48                                   # 4.0
    table = np.array([[0, 1]], np.int32)
    ind = np.array([[1, 6, 2]], np.int32)                  # token 1 (page 0), 6 (page 1)
    q = np.zeros((1, 2, D), np.uint16)
    q[0, :, 0] = _bf16_bits(np.array([1.0]))[0]
    gate = np.zeros((1, 2, D), np.uint16)
    slots = orc.qsa_slots(ind, table, np.zeros(1, np.int32), 2, page)
    out, _ = orc.qsa_decode(q, k, v, slots, ind, orc.qsa_offset_bits(page), math.log(3.0),
                            1.0, gate)
    np.testing.assert_allclose(out, np.full((1, 2, D), 0.5 * (0.75 * 2.0 + 0.25 * 4.0)),
                               rtol=1e-15)


@pytest.mark.parametrize("combined", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (4, 4), (8, 1)])
def test_qsa_matches_torch_sdpa_on_tokens_gathered_from_logical_indices(Hq, Hkv, combined):
    """Grouped-query attention of torch.nn.functional.scaled_dot_product_attention in
    float64 on K/V rows gathered straight from the logical indices and the block table
    (not through the slots), times output_scale and sigmoid(gate).  Duplicated and -1
    entries, and entries past the valid count, are in the selection."""
    rng = np.random.default_rng(100 + Hq * 7 + Hkv + (50 if combined else 0))
    c = _qsa_case(rng, Hq=Hq, Hkv=Hkv, combined=combined)
    ind = c["ind"].copy()
    ind[:, 3] = ind[:, 1]                                   # a duplicate
    ind[:, 4] = -1                                          # a masked entry
    ind[:, -2] = ind[:, 0]                                  # past the count: ignored
    out, _ = _qsa_run(c, softmax_scale=0.21, output_scale=1.3, ind=ind)
    for r in range(ind.shape[0]):
        n = ind[r, -1]
        toks = [x for x in ind[r, :n] if x >= 0]
        pages = c["table"][r, [x // c["page"] for x in toks]]
        places = [x % c["page"] for x in toks]
        kk = _e4m3_values(c["k"][pages, places])           # [n, Hkv, D]
        vv = _e4m3_values(c["v"][pages, places])
        qq = torch.from_numpy(_bf16_values(c["q"][r]))[:, None, :]          # [Hq, 1, D]
        att = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.from_numpy(kk).transpose(0, 1), torch.from_numpy(vv).transpose(0, 1),
            scale=0.21, enable_gqa=True)[:, 0, :].numpy()
        want = 1.3 * att * _sigmoid(_bf16_values(c["gate"][r]))
        np.testing.assert_allclose(out[r], want, rtol=1e-12, atol=1e-14)


def test_qsa_selection_invariants():
    """Reordering the selected columns changes nothing (up to double rounding); a row with
    count 0, a negative count or only -1 entries outputs zeros; a count above topk is
    clipped to topk."""
    rng = np.random.default_rng(13)
    c = _qsa_case(rng)
    base, _ = _qsa_run(c)
    ind = c["ind"].copy()
    for r in range(ind.shape[0]):
        n = ind[r, -1]
        ind[r, :n] = ind[r, :n][rng.permutation(n)]
    perm, _ = _qsa_run(c, ind=ind)
    np.testing.assert_allclose(perm, base, rtol=1e-13, atol=1e-15)
    ind = c["ind"].copy()
    ind[0, -1] = 0
    ind[1, -1] = -3
    ind[2, :-1] = -1
    z, _ = _qsa_run(c, ind=ind)
    assert not z.any()
    ind = c["ind"].copy()
    big = ind.copy()
    big[:, -1] = 1000                      # clipped to topk: the -1 padding is masked anyway
    a, _ = _qsa_run(c, ind=big)
    b, _ = _qsa_run(c, ind=ind)
    np.testing.assert_array_equal(a, b)


def test_qsa_tolbase_bounds_the_output():
    rng = np.random.default_rng(14)
    c = _qsa_case(rng)
    out, tb = _qsa_run(c, output_scale=-0.5)
    assert np.all(np.abs(out) <= tb * (1 + 1e-12))
    assert np.all(tb > 0)
