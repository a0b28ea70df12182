"""GPU parity of fp4idx_logits_topk_paged (scores and top-k without writing the logits).

Fewer than 512 rows go through the logits (in the workspace) and the plain top-k; 512
or more take the sampled-threshold path, whose cases below use 560-600 rows.

Against the oracle: the chosen column sets equal the oracle's top-k of its own logits,
except for columns whose oracle scores tie with the oracle's k-th within the logits
tolerance (1e-6 of the summed |w ReLU(dot)| of both columns), as for the unfused path.
Against the unfused GPU path (logits_paged + topk on the same inputs): indices and
values equal bit for bit -- the fused scorer computes the same fp32 scores.
"""
import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def _args(case):
    return (dev(case.q_fp4), dev(case.q_scale), dev(case.w), dev(case.k_fp4), dev(case.k_scale),
            dev(case.block_table), dev(case.cu_seqlens_q), dev(case.row_lens))


def _fused(case, k, out_cols=None):
    out_cols = case.out_cols if out_cols is None else out_cols
    say(f"[gpu] logits_topk {case.name} T={case.T} H={case.H} Hkv={case.Hkv} B={case.B} "
        f"page={case.page_size} out_cols={out_cols} k={k} fmt={case.fmt}")
    idx, vals = fp4.logits_topk_paged(*_args(case), fmt=case.fmt, out_cols=out_cols, k=k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


def _unfused(case, k, out_cols=None):
    out_cols = case.out_cols if out_cols is None else out_cols
    a = _args(case)
    logits = fp4.logits_paged(*a, fmt=case.fmt, out_cols=out_cols)
    idx, vals = fp4.topk(logits, k, a[7])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


def _check_oracle(case, gidx, k, rows=None, out_cols=None):
    """Tie-tolerant comparison with the oracle's top-k of its own logits."""
    out_cols = case.out_cols if out_cols is None else out_cols
    rows = np.arange(case.T) if rows is None else np.asarray(rows)
    ref, tb, inexact = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                        case.k_scale, case.block_table, case.cu_seqlens_q,
                                        case.row_lens, case.page_size, out_cols, rows=rows,
                                        want_tolbase=True, compact=True)
    assert inexact == 0
    oi, _ = orc.topk(ref, k, np.minimum(case.row_lens[rows], out_cols))
    ndiff = 0
    for i, t in enumerate(rows.tolist()):
        g = gidx[t]
        a, b = set(g[g >= 0].tolist()), set(oi[i][oi[i] >= 0].tolist())
        assert len(a) == len(b), (t, len(a), len(b))
        assert np.all(g[len(a):] == -1) and np.all(np.diff(g[:len(a)]) > 0)
        if not b:
            continue
        sel = np.array(sorted(b))
        kcol = sel[np.argmin(ref[i][sel])]
        for c in a ^ b:
            gap = abs(float(ref[i, c]) - float(ref[i, kcol]))
            assert gap <= 1e-6 * (float(tb[i, c]) + float(tb[i, kcol])) + 1e-30, (t, c)
        ndiff += len(a ^ b)
    say(f"    {rows.size} rows match the oracle (symmetric differences within tolerance: {ndiff})")


def _check_unfused(case, gi, gv, k, out_cols=None):
    ui, uv = _unfused(case, k, out_cols)
    np.testing.assert_array_equal(gi, ui)
    np.testing.assert_array_equal(gv.view(np.uint32), uv.view(np.uint32))


@pytest.mark.parametrize("spec", [
    dict(q_per_req=[4], ctx=[2048], H=32, k=256),
    dict(q_per_req=[3, 1, 5], ctx=[9000, 300, 5000], H=32, k=512),
    dict(q_per_req=[2, 2], ctx=[20000, 12000], H=64, k=2048),
    dict(q_per_req=[1, 1, 1, 1, 1], ctx=[70, 1, 4100, 2049, 2047], H=16, k=2048),
    dict(q_per_req=[4], ctx=[3000], H=32, Hkv=4, k=64),
    dict(q_per_req=[2, 3], ctx=[5000, 700], H=32, k=1, page=128),
    dict(q_per_req=[4, 4], ctx=[6000, 6000], H=32, k=300, fmt=wl.NVFP4),
])
def test_small_cases(spec):
    spec = dict(spec)
    k = spec.pop("k")
    seed = sum(spec["ctx"]) + k
    case = wl.make_logits("fused", seed=seed, **spec)
    gi, gv = _fused(case, k)
    _check_oracle(case, gi, k)
    _check_unfused(case, gi, gv, k)


def test_config0_and_output_wider_than_rows():
    case = wl.config0()
    gi, gv = _fused(case, 2048, out_cols=2048 + 640)
    _check_oracle(case, gi, 2048, out_cols=2048 + 640)
    _check_unfused(case, gi, gv, 2048, out_cols=2048 + 640)


@pytest.mark.parametrize("ctx", [16384, 100_000])
def test_config1_decode(ctx):
    case = wl.config1(ctx)
    gi, gv = _fused(case, 2048)
    _check_oracle(case, gi, 2048)
    _check_unfused(case, gi, gv, 2048)


def test_sample_defeated_rows_take_the_second_pass():
    """Keys on the sampled pages (logical pages 0, 16, 32, ...) get scales 2^8 above the
    rest, so every row's top 2048 lies on sampled pages and the threshold from the sample
    (its 256th largest score) is reached by only about 256 scores of the row: the first
    selection cannot be exact and the second pass must produce the result.  Request 1
    keeps plain keys (its rows stay on the first pass)."""
    case = wl.make_logits("defeat", q_per_req=[4, 4], ctx=[60000, 50000], H=32, seed=77)
    case.k_scale[...] = 123
    W = case.block_table.shape[1]
    for lp in range(0, W, 16):
        ph = case.block_table[0, lp]
        if ph >= 0:
            case.k_scale[ph] = 131
    gi, gv = _fused(case, 2048)
    _check_oracle(case, gi, 2048)
    _check_unfused(case, gi, gv, 2048)


def test_invalid_pages_and_rows_outside_requests():
    case = wl.make_logits("holes", q_per_req=[3, 3], ctx=[8000, 6000], H=32, seed=12)
    case.block_table[0, 5] = -1
    case.block_table[1, 2] = case.k_fp4.shape[0] + 3
    case.cu_seqlens_q[-1] -= 1                       # the last row belongs to no request
    gi, gv = _fused(case, 1024)
    _check_oracle(case, gi, 1024, rows=np.arange(case.T - 1))
    assert np.all(gi[-1] == -1) and np.all(gv[-1] == -np.inf)   # a row of no request
    _check_unfused(case, gi, gv, 1024)


def test_config2_batched_sampled_rows():
    case = wl.config2()
    gi, gv = _fused(case, 2048)
    rng = np.random.default_rng(1021)
    rows = np.sort(rng.choice(case.T, 6, replace=False))
    _check_oracle(case, gi, 2048, rows=rows)
    _check_unfused(case, gi, gv, 2048)


def test_config4_prefill_sampled_rows():
    case = wl.config4()
    gi, gv = _fused(case, 2048)
    rng = np.random.default_rng(1041)
    rows = np.unique(np.concatenate([rng.choice(case.T, 24, replace=False),
                                     [0, 2046, 2047, 2048, 32767]]))
    _check_oracle(case, gi, 2048, rows=rows)
    ui, uv = _unfused(case, 2048)
    np.testing.assert_array_equal(gi, ui)
    np.testing.assert_array_equal(gv.view(np.uint32), uv.view(np.uint32))


# ---- the sampled-threshold path (512 rows or more)

def test_sampled_path_many_rows():
    case = wl.make_logits("fused_many", q_per_req=[300, 260], ctx=[9000, 5000], H=32, seed=91)
    gi, gv = _fused(case, 512)
    _check_oracle(case, gi, 512, rows=[0, 1, 150, 299, 300, 301, 559])
    _check_unfused(case, gi, gv, 512)


def test_sampled_path_defeated_rows_take_the_second_pass():
    """As test_sample_defeated_rows_take_the_second_pass, with enough rows for the
    sampled-threshold path: request 0's largest scores all lie on sampled pages."""
    case = wl.make_logits("defeat_many", q_per_req=[300, 300], ctx=[60000, 50000], H=32, seed=78)
    case.k_scale[...] = 123
    W = case.block_table.shape[1]
    for lp in range(0, W, 16):
        ph = case.block_table[0, lp]
        if ph >= 0:
            case.k_scale[ph] = 131
    gi, gv = _fused(case, 2048)
    _check_oracle(case, gi, 2048, rows=[0, 5, 299, 300, 599])
    _check_unfused(case, gi, gv, 2048)


def test_sampled_path_invalid_pages_and_rows_outside_requests():
    case = wl.make_logits("holes_many", q_per_req=[300, 300], ctx=[8000, 6000], H=32, seed=13)
    case.block_table[0, 5] = -1
    case.block_table[1, 2] = case.k_fp4.shape[0] + 3
    case.cu_seqlens_q[-1] -= 1                       # the last row belongs to no request
    gi, gv = _fused(case, 1024)
    _check_oracle(case, gi, 1024, rows=[0, 1, 299, 300, 598])
    assert np.all(gi[-1] == -1) and np.all(gv[-1] == -np.inf)
    _check_unfused(case, gi, gv, 1024)


def test_sampled_path_one_row_per_request():
    """520 requests of one row each: the sampled-threshold path with one-row blocks
    (two waves per scorer workgroup), contexts from 300 to 5000 keys."""
    rng = np.random.default_rng(93)
    ctx = rng.integers(300, 5000, 520).tolist()
    case = wl.make_logits("fused_one_row", q_per_req=[1] * 520, ctx=ctx, H=64, seed=94)
    gi, gv = _fused(case, 1024)
    _check_oracle(case, gi, 1024, rows=[0, 1, 2, 259, 518, 519])
    _check_unfused(case, gi, gv, 1024)
