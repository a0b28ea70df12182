"""GPU parity of fp4idx_block_scores against the CPU oracle.

MXFP4 block maxima are maxima of single scaled-FP4 MFMA results, which add their four
exact 32-element block sums in fp32: bit-exact unless one of those three additions
rounds (rare at scale codes 123..131; the exact fraction is reported and must stay
above 99%), and within 2^-22 * sum_d |q_d k_d| over the block's keys (errbase).  NVFP4
accumulates four fp16 MFMAs in fp32, held to 2^-17 * errbase (one rounding per
addition over 128 products; see DOT_BOUND).  The -inf pattern must match exactly.
"""
import numpy as np
import pytest

from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import DOT_BOUND, gpu_block_scores, oracle_block_scores, say

pytestmark = pytest.mark.gpu


def _check(case, rows=None, exact=False, nan_codes=False):
    """exact=True: at least 99% of the visible block maxima are bit-exact.
    nan_codes=True: the case holds NaN scale codes, whose dots the oracle cannot call
    exact (they are NaN and skipped by the max)."""
    got = gpu_block_scores(case)
    ref, eb, inexact = oracle_block_scores(case, rows=rows)
    assert nan_codes or inexact == 0
    cols = np.arange(case.Tq) if rows is None else np.asarray(rows)
    g, r, e = got[:, :, cols], ref[:, :, cols], eb[:, :, cols]
    inv = r == -np.inf
    assert np.array_equal(g == -np.inf, inv)
    vis = ~inv
    diff = np.abs(g[vis].astype(np.float64) - r[vis])
    n_exact = int((g[vis] == r[vis]).sum())
    worst = float((diff / (2.0 ** -24 * np.maximum(e[vis], 1e-30))).max()) if diff.size else 0.0
    say(f"    bit-exact {n_exact}/{int(vis.sum())}, worst error {worst:.2f} * 2^-24 * errbase")
    if exact:
        assert n_exact >= 0.99 * int(vis.sum())
    assert np.all(diff <= DOT_BOUND[case.fmt] * e[vis])


CASES = [
    dict(name="mx_causal", fmt=wl.MXFP4, q_lens=[5, 130, 1], k_lens=[300, 130, 129], Hq=8, Hkv=2,
         causal=True),
    dict(name="mx_noncausal", fmt=wl.MXFP4, q_lens=[17, 3], k_lens=[257, 128], Hq=4, Hkv=1,
         causal=False),
    dict(name="mx_qo_offset", fmt=wl.MXFP4, q_lens=[20, 33], k_lens=[200, 90], Hq=16, Hkv=1,
         causal=True, qo_offset=[7, -5]),
    dict(name="mx_gqa17", fmt=wl.MXFP4, q_lens=[9], k_lens=[257], Hq=17, Hkv=1, causal=True),
    dict(name="nv_causal", fmt=wl.NVFP4, q_lens=[5, 130, 1], k_lens=[300, 130, 129], Hq=8, Hkv=2,
         causal=True),
    dict(name="nv_noncausal", fmt=wl.NVFP4, q_lens=[4, 8], k_lens=[128, 257], Hq=4, Hkv=1,
         causal=False),
    dict(name="nv_qo_offset", fmt=wl.NVFP4, q_lens=[20], k_lens=[400], Hq=32, Hkv=4, causal=True,
         qo_offset=[100]),
    dict(name="nv_q_longer_than_k", fmt=wl.NVFP4, q_lens=[40], k_lens=[20], Hq=4, Hkv=2,
         causal=True),
]


@pytest.mark.parametrize("spec", CASES, ids=[c["name"] for c in CASES])
def test_small_cases(spec):
    spec = dict(spec)
    name = spec.pop("name")
    case = wl.make_block(name, seed=len(name) * 31, **spec)
    _check(case, exact=spec["fmt"] == wl.MXFP4)


def test_ktiles_wider_than_batch_and_bad_pages():
    case = wl.make_block("wide", fmt=wl.MXFP4, q_lens=[6, 6], k_lens=[140, 600], Hq=4, Hkv=1,
                         seed=3, causal=False)
    case.max_seqlen_k = 1000          # more output blocks than any batch item fills
    case.kv_indices[1] = -1           # batch 0, block 1 has no page
    _check(case, exact=True)


def test_nvfp4_nan_scale_codes_are_skipped_by_the_max():
    """A NaN E4M3 code makes every dot it touches NaN; max is C's fmax on both sides, so
    those dots are skipped (a query head whose dots are all NaN gives -inf blocks)."""
    case = wl.make_block("nv_nan", fmt=wl.NVFP4, q_lens=[6, 3], k_lens=[300, 129], Hq=4, Hkv=2,
                         seed=77, causal=False)
    case.q_scale[2, 1, 3] = 0x7F               # query row 2, head 1: all its dots NaN
    case.q_scale[7, 3, 0] = 0xFF               # query row 7 (batch 1), head 3
    p0 = int(case.kv_indices[case.cu_page_offsets[0]])
    case.k_scale[p0, 0, 5, 2] = 0x7F            # one key of batch 0, key head 0
    _check(case, nan_codes=True)


def test_nvfp4_shared_decoding_noncausal_bad_pages_and_head_groups():
    """NVFP4 workgroups whose 64 tokens lie in one batch item share their key decoding;
    the one that straddles items 1 and 2 decodes per wave.  Non-causal items of 64 or
    more tokens, a missing page and one outside the cache, more output blocks than any
    item fills, six query heads per key head (the second head group of each key head is
    partial) and a NaN key scale inside a shared block."""
    case = wl.make_block("nv_shared", fmt=wl.NVFP4, q_lens=[64, 100, 70], k_lens=[700, 1500, 260],
                         Hq=12, Hkv=2, seed=5, causal=False)
    case.max_seqlen_k = 1800
    o1 = int(case.cu_page_offsets[1])
    case.kv_indices[o1 + 3] = -1
    case.kv_indices[o1 + 5] = case.k_fp4.shape[0] + 2
    p0 = int(case.kv_indices[1])
    case.k_scale[p0, 1, 7, 3] = 0x7F
    _check(case, nan_codes=True)


def test_nvfp4_shared_decoding_long_keys_with_offset():
    """One causal item whose 130 tokens see 8801..8930 keys (past 64 blocks, so the
    block-table window moves, and across several key chunks), through qo_offset."""
    case = wl.make_block("nv_long", fmt=wl.NVFP4, q_lens=[130], k_lens=[9000], Hq=8, Hkv=1,
                         seed=6, causal=True, qo_offset=[8800])
    _check(case, rows=[0, 1, 17, 63, 64, 65, 100, 127, 128, 129])


def test_config3_nvfp4_prefill_sampled_queries():
    case = wl.config3()
    rng = np.random.default_rng(1030)
    # 256 sampled query tokens plus the first, second, last and second-to-last of
    # every batch item
    rows = np.unique(np.concatenate([rng.choice(case.Tq, 256, replace=False),
                                     case.cu_seqlens_q[:-1], case.cu_seqlens_q[:-1] + 1,
                                     case.cu_seqlens_q[1:] - 1, case.cu_seqlens_q[1:] - 2]))
    _check(case, rows=rows.tolist())
