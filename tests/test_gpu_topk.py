"""GPU parity of fp4idx_topk.

On the same scores the selection is integer work and must equal the oracle's exactly
(columns in increasing order, -1 padding, values copied from the scores).  On logits
that the GPU and the oracle each computed, the index sets may differ only where the
oracle's scores tie within the logits tolerance.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import gpu_logits, gpu_topk, oracle_logits, say

pytestmark = pytest.mark.gpu


def _same(scores, k, row_lens=None):
    gi, gv = gpu_topk(scores, k, row_lens)
    oi, ov = orc.topk(scores, k, row_lens)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("rows,cols,k", [(4, 2048, 2048), (4, 5000, 2048), (3, 32768, 2048),
                                         (2, 32769, 100), (4, 100_000, 2048), (2, 400_000, 2048),
                                         (64, 131072, 2048), (7, 70_000, 8192), (5, 1000, 1)])
def test_same_scores_exact(rows, cols, k):
    rng = np.random.default_rng(rows * 7 + cols)
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0, rng.integers(0, cols, 50)] = -np.inf
    s[-1, rng.integers(0, cols, 50)] = np.nan
    _same(s, k)


@pytest.mark.parametrize("rows,cols", [(4, 100_000), (3, 20_000)])
def test_indices_only(rows, cols):
    """out_vals NULL: the same indices, and no value is read back."""
    import sparse_attention_fp4_amd as fp4
    from .gpu_helpers import dev

    rng = np.random.default_rng(cols)
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = np.array([cols - 3 * i for i in range(rows)], np.int32)
    say(f"[gpu] topk indices only rows={rows} cols={cols}")
    idx, vals = fp4.topk(dev(s), 2048, dev(lens), want_vals=False)
    assert vals is None
    oi, _ = orc.topk(s, 2048, lens)
    assert np.array_equal(idx.cpu().numpy(), oi)


@pytest.mark.parametrize("cols", [40000, 20000, 3000])
def test_ties_zeros_and_lengths(cols):
    rng = np.random.default_rng(4)
    rows, k = 6, 2048
    s = (rng.integers(-20, 20, (rows, cols)) / 4).astype(np.float32)  # heavy ties
    s[1, ::3] = -0.0
    s[2, :] = 1.5                                                     # all equal
    s[3, :] = -np.inf                                                 # nothing valid
    s[4, 100:] = -np.inf                                              # fewer than k valid
    lens = np.array([cols, cols - 1, 1, cols // 2, cols, 0], np.int32)
    _same(s, k, lens)


@pytest.mark.parametrize("cols", [16384, 100_000])
def test_clustered_values_with_outliers(cols):
    """Most scores in a narrow band, a few far away (value-space bins put nearly all in
    one bin), plus +inf entries."""
    rng = np.random.default_rng(cols + 1)
    s = (1.0 + rng.standard_normal((3, cols)) * 1e-6).astype(np.float32)
    s[0, 7] = 1e30
    s[0, 9] = -1e30
    s[1, 100] = np.inf
    s[2, :] = np.float32(1.0)
    s[2, ::17] = np.float32(1.0000001)
    _same(s, 2048)


def test_on_config1_logits_within_tie_tolerance():
    case = wl.config1(100_000)
    got = gpu_logits(case)
    ref, tb, _ = oracle_logits(case)
    gi, _ = gpu_topk(got, 2048, case.row_lens)
    oi, _ = orc.topk(ref, 2048, case.row_lens)
    for t in range(case.T):
        a, b = set(gi[t][gi[t] >= 0]), set(oi[t][oi[t] >= 0])
        assert len(a) == len(b) == min(2048, case.row_lens[t])
        sel = np.array(sorted(b))
        kcol = sel[np.argmin(ref[t][sel])]        # the oracle's k-th largest
        for c in a ^ b:
            gap = abs(float(ref[t, c]) - float(ref[t, kcol]))
            assert gap <= 1e-6 * (float(tb[t, c]) + float(tb[t, kcol])) + 1e-30, c
        say(f"    row {t}: symmetric difference {len(a ^ b)}")


def test_long_rows_largest_keys_crowded_into_one_chunk():
    """Long rows whose largest scores crowd into one 4096-column stretch instead of
    spreading along the row: 4000 raised scores in one stretch, 3000 equal largest
    scores (ties at the k-th), exactly k raised scores in one stretch, and a plain row."""
    rng = np.random.default_rng(31)
    rows, cols, k = 4, 100_000, 2048
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0, 8192:8192 + 4000] += 10.0
    s[1, :3000] = 50.0
    s[2, 50_000:50_000 + k] = (9.0 + rng.random(k)).astype(np.float32)
    say(f"[gpu] topk crowded chunks rows={rows} cols={cols} k={k}")
    _same(s, k)


def test_long_rows_all_equal_and_mixed_lengths():
    """A row of equal scores (all ties: the first k columns win) next to rows of lengths
    0, 1, k - 1, k, k + 1 and 3000, in a batch wider than 32768 columns."""
    rng = np.random.default_rng(32)
    rows, cols, k = 8, 200_000, 2048
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0] = 1.5
    lens = np.array([cols, cols, 0, 1, k - 1, k, k + 1, 3000], np.int32)
    say(f"[gpu] topk equal scores and lengths rows={rows} cols={cols} k={k}")
    _same(s, k, lens)


@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_long_rows_k_sizes(k):
    rng = np.random.default_rng(40 + k)
    rows, cols = 3, 150_000
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0, rng.integers(0, cols, 500)] = -np.inf
    s[1, rng.integers(0, cols, 500)] = np.nan
    lens = np.array([cols, cols - 17, 33_000], np.int32)
    say(f"[gpu] topk long rows k={k}")
    _same(s, k, lens)


@pytest.mark.parametrize("extra", [80, 1500])
def test_long_rows_one_chunk_overflowing_its_slots(extra):
    """One 4096-column chunk holds `extra` more keys of the threshold's digit bin than the
    rest: 80 overflow its up-front candidate slots but fit wider ones, 1500 need the
    round-by-round reads."""
    rng = np.random.default_rng(90 + extra)
    rows, cols, k = 3, 100_000, 2048
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    for r in range(rows):
        t = np.sort(s[r])[-k]
        s[r, 5 * 4096:5 * 4096 + extra] = (t * (1 + 1e-4 * rng.standard_normal(extra))).astype(np.float32)
    say(f"[gpu] topk overflowing chunk extra={extra}")
    _same(s, k)


def test_many_long_rows_of_mixed_lengths():
    """64 rows of up to 131072 columns with lengths spread like batched decode (several
    chunks per histogram and finishing workgroup, chunks past a row's end skipped),
    plus rows of length 0, 1, k and k + 1 and a row of ties."""
    rng = np.random.default_rng(77)
    rows, cols, k = 64, 131_072, 2048
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[5] = (rng.integers(-8, 8, cols) / 2).astype(np.float32)
    lens = rng.integers(4096, cols + 1, rows).astype(np.int32)
    lens[:4] = [0, 1, k, k + 1]
    lens[4] = cols
    say(f"[gpu] topk many long rows rows={rows} cols={cols} k={k}")
    _same(s, k, lens)


@pytest.mark.parametrize("rows,cols", [(64, 8193), (65, 8193), (64, 8192), (1, 32768), (511, 32768)])
def test_routing_boundaries(rows, cols):
    """Both sides of the routing between one workgroup per row and the chunked path
    (more than 8192 columns and at most 64 rows go to the chunked path)."""
    rng = np.random.default_rng(rows * 3 + cols)
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0, rng.integers(0, cols, 40)] = -np.inf
    lens = rng.integers(0, cols + 1, rows).astype(np.int32)
    lens[0] = cols
    say(f"[gpu] topk routing rows={rows} cols={cols}")
    _same(s, 2048, lens)


def test_workspace_reused_across_calls_without_clearing():
    """The long-row path leaves its workspace ready for the next call."""
    import torch

    import sparse_attention_fp4_amd as fp4
    from .gpu_helpers import dev

    rng = np.random.default_rng(8)
    rows, cols, k = 3, 70_000, 2048
    ws = torch.zeros(fp4.topk_workspace_bytes(rows, cols, k), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        s = rng.standard_normal((rows, cols)).astype(np.float32) * (rep + 1)
        lens = np.array([cols, cols - 5 * rep, 40_000], np.int32)
        say(f"[gpu] topk workspace reuse {rep}")
        idx, vals = fp4.topk(dev(s), k, dev(lens), workspace=ws)
        oi, ov = orc.topk(s, k, lens)
        assert np.array_equal(idx.cpu().numpy(), oi)
        assert np.array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("rows,cols,k,kind", [(4, 32_768, 2048, "normal"), (6, 20_000, 2048, "ties"),
                                              (2, 30_000, 7, "normal"), (3, 16_384, 2048, "clustered"),
                                              (8, 9_000, 8192, "normal"), (20, 12_000, 2048, "normal"),
                                              (4, 50_000, 2048, "normal"), (64, 70_000, 2048, "ties")])
def test_few_long_rows_when_the_waits_run_out(rows, cols, k, kind):
    """Up to 64 rows of 8193..53248 columns (and 48 to 64 rows of up to 131072 columns)
    take one kernel whose workgroups wait for each other; with the wait bound at 0 polls
    every row with more than one chunk is recomputed by one workgroup from its scores
    (the path taken when a row's workgroups cannot all run at once), and the result is
    the same.  The workspace is then ready for a normal call."""
    import torch

    import sparse_attention_fp4_amd as fp4
    from .gpu_helpers import dev

    rng = np.random.default_rng(rows + cols + k)
    if kind == "ties":
        s = (rng.integers(-20, 20, (rows, cols)) / 4).astype(np.float32)
        s[1, ::3] = -0.0
        s[2, :] = 1.5
        s[3, :] = -np.inf
    elif kind == "clustered":
        s = (1.0 + rng.standard_normal((rows, cols)) * 1e-6).astype(np.float32)
        s[0, 5] = np.inf
    else:
        s = rng.standard_normal((rows, cols)).astype(np.float32)
        s[0, rng.integers(0, cols, 50)] = -np.inf
        s[-1, rng.integers(0, cols, 50)] = np.nan
    lens = np.full(rows, cols, np.int32)
    lens[-1] = 0 if rows > 4 else cols - 4097
    if rows > 4:
        lens[-2] = 1
    ws = torch.zeros(fp4.topk_workspace_bytes(rows, cols, k), dtype=torch.uint8, device="cuda")
    oi, ov = orc.topk(s, k, lens)
    prev = fp4.ops.set_topk_wait_limit(0)
    try:
        say(f"[gpu] topk waits run out rows={rows} cols={cols} k={k} {kind}")
        idx, vals = fp4.topk(dev(s), k, dev(lens), workspace=ws)
        torch.cuda.synchronize()
    finally:
        fp4.ops.set_topk_wait_limit(prev)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))
    say("[gpu] topk after the fallback, same workspace")
    idx, vals = fp4.topk(dev(s), k, dev(lens), workspace=ws)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("many", [False, True], ids=["16x32768", "64x131072"])
def test_one_kernel_rows_beside_other_work_on_the_gpu(many):
    """The one-kernel route while a large matrix product runs on another stream: the
    rows' workgroups may not all be resident at first (their waits are bounded, and a
    wait that runs out has the row recomputed), so the result is the same either way.
    Repeated with the wait bound at 200 polls, where running out is likely."""
    import torch

    import sparse_attention_fp4_amd as fp4
    from .gpu_helpers import dev

    rng = np.random.default_rng(71)
    rows, cols, k = 16, 32_768, 2048
    if many:
        rows, cols = 64, 131_072
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = rng.integers(1, cols + 1, rows).astype(np.int32)
    lens[0] = cols
    oi, _ = orc.topk(s, k, lens)
    ds, dl = dev(s), dev(lens)
    ws = torch.zeros(fp4.topk_workspace_bytes(rows, cols, k), dtype=torch.uint8, device="cuda")
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    other = torch.cuda.Stream()
    torch.cuda.synchronize()
    for limit in (None, 200):
        prev = fp4.ops.set_topk_wait_limit(limit) if limit is not None else None
        try:
            for rep in range(3):
                say(f"[gpu] topk beside a matmul, wait bound {limit}, call {rep}")
                with torch.cuda.stream(other):
                    c = a @ b
                idx, _ = fp4.topk(ds, k, dl, want_vals=False, workspace=ws)
                torch.cuda.synchronize()
                assert np.array_equal(idx.cpu().numpy(), oi)
                del c
        finally:
            if prev is not None:
                fp4.ops.set_topk_wait_limit(prev)


def test_workspace_reused_per_shape_and_cleared_between_shapes():
    """One allocation serves calls of 4 rows (one kernel, in-memory waits) and of 64
    rows (three kernels): calls of one shape reuse it without clearing, and it is
    zero-filled when the shape changes (the layout depends on the shape)."""
    import torch

    import sparse_attention_fp4_amd as fp4
    from .gpu_helpers import dev

    rng = np.random.default_rng(12)
    cols, k = 32_768, 2048
    nb = max(fp4.topk_workspace_bytes(r, cols, k) for r in (4, 64))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for rep, rows in enumerate((4, 4, 64, 64, 4, 4)):
        if rep in (2, 4):
            ws.zero_()
        s = rng.standard_normal((rows, cols)).astype(np.float32)
        lens = rng.integers(1, cols + 1, rows).astype(np.int32)
        lens[0] = cols
        say(f"[gpu] topk workspace call {rep} rows={rows}")
        idx, _ = fp4.topk(dev(s), k, dev(lens), workspace=ws, want_vals=False)
        oi, _ = orc.topk(s, k, lens)
        assert np.array_equal(idx.cpu().numpy(), oi)


@pytest.mark.parametrize("rows,cols", [(8, 32_768), (27, 32_768), (32, 32_768), (64, 16_384), (45, 12_000),
                                       (16, 53_248), (48, 100_000), (47, 100_000), (24, 131_072),
                                       (40, 100_000)])
def test_few_rows_in_one_kernel_lengths_and_ties(rows, cols):
    """Rows in one kernel (up to 13 chunk workgroups of 4096 columns a row and 32 a die,
    or, for many rows, up to 8 of 16384 columns, one a CU up to 32 rows and two from 48;
    40 and 47 rows of 100000 take the three kernels): a row of equal scores, rows of
    lengths 0, 1, k - 1, k, k + 1 and 5000, and heavy ties."""
    rng = np.random.default_rng(33 + rows)
    k = 2048
    s = (rng.integers(-40, 40, (rows, cols)) / 8).astype(np.float32)
    s[0] = 1.5
    s[1, rng.integers(0, cols, 300)] = np.nan
    lens = np.full(rows, cols, np.int32)
    lens[:8] = [cols, cols - 1, 0, 1, k - 1, k, k + 1, 5000]
    lens[8:] = rng.integers(1, cols + 1, rows - 8)
    say(f"[gpu] topk one kernel lengths and ties rows={rows} cols={cols} k={k}")
    _same(s, k, lens)


def _sampled_columns(length):
    """128 runs of 32 columns at run starts floor(r * length / 128) rounded down to a
    multiple of 32 (the whole row when it has at most 4096 columns): a fixed 4% sample
    that a sampled threshold could be placed from."""
    if length <= 4096:
        return np.arange(length)
    starts = ((np.arange(128, dtype=np.int64) * length) // 128) & ~31
    return (starts[:, None] + np.arange(32)[None, :]).ravel()


@pytest.mark.parametrize("rows,cols,k", [(3, 100_000, 2048), (2, 40_000, 300), (70, 40_000, 2048)])
def test_long_rows_where_the_sample_misjudges(rows, cols, k):
    """Rows whose largest scores sit on a regular 4% sample of the columns (a threshold
    placed from that sample would let through far fewer than k keys), and a row whose
    largest scores lie only off it: the selection is exact regardless."""
    rng = np.random.default_rng(rows + cols + k)
    s = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = np.full(rows, cols, np.int32)
    lens[-1] = cols - 777
    for r in range(rows):
        samp = _sampled_columns(int(lens[r]))
        if r == 1:
            off = np.setdiff1d(np.arange(lens[r]), samp)
            s[r, off[rng.choice(off.size, 3 * k, replace=False)]] += 20.0
        else:
            s[r, samp] += 20.0
    say(f"[gpu] topk sample-defeating rows rows={rows} cols={cols} k={k}")
    _same(s, k, lens)


@pytest.mark.parametrize("rows,cols,k,kind", [(600, 4096, 2048, "normal"), (520, 32768, 2048, "ties"),
                                              (512, 20000, 100, "clustered"), (700, 3000, 2048, "normal")])
def test_many_short_rows(rows, cols, k, kind):
    """Many rows of <= 32768 columns take one streaming workgroup per row."""
    rng = np.random.default_rng(rows + cols + k)
    say(f"[gpu] topk many rows rows={rows} cols={cols} k={k} {kind}")
    if kind == "ties":
        s = (rng.integers(-20, 20, (rows, cols)) / 4).astype(np.float32)
    elif kind == "clustered":
        s = (1.0 + rng.standard_normal((rows, cols)) * 1e-6).astype(np.float32)
    else:
        s = rng.standard_normal((rows, cols)).astype(np.float32)
    s[0, rng.integers(0, cols, 50)] = -np.inf
    s[1, rng.integers(0, cols, 50)] = np.nan
    s[2, :] = -np.inf
    lens = rng.integers(0, cols + 1, rows).astype(np.int32)
    lens[:6] = [cols, cols, cols, 0, 1, min(cols, k)]
    _same(s, k, lens)
