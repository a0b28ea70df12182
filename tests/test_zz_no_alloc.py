"""fp4idx_logits_topk_paged_noalloc (static per-GPU scratch, nothing allocated) against
fp4idx_logits_topk_paged with a caller workspace: indices and values equal bit for bit,
on calls in a row whose sizes shrink (so a later call meets what an earlier one left in
the scratch), through both routes of the fused entry point, called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_attention_fp4_amd import _lib
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def _call(case, k, noalloc):
    L = _lib.lib()
    q, qs, w, kf, ks = (dev(a) for a in (case.q_fp4, case.q_scale, case.w, case.k_fp4, case.k_scale))
    bt, cu, lens = dev(case.block_table), dev(case.cu_seqlens_q), dev(case.row_lens)
    T, H, Hkv, page, P = case.T, case.H, case.Hkv, case.page_size, case.num_pages
    G = wl.groups(case.fmt)
    W = case.block_table.shape[1]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    vals = torch.full((T, k), np.nan, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    head = (case.fmt, q.data_ptr(), H * 64, qs.data_ptr(), H * G, w.data_ptr(), H,
            kf.data_ptr(), Hkv * page * 64, ks.data_ptr(), Hkv * page * G, bt.data_ptr(), W,
            cu.data_ptr(), lens.data_ptr(), T, case.B, H, Hkv, page, P, W, case.out_cols, k,
            idx.data_ptr(), vals.data_ptr())
    if noalloc:
        rc = L.fp4idx_logits_topk_paged_noalloc(*head, stream)
        name = "fp4idx_logits_topk_paged_noalloc"
    else:
        need = L.fp4idx_logits_topk_workspace_bytes(case.fmt, T, case.B, H, Hkv, page, W,
                                                    case.out_cols, k)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc = L.fp4idx_logits_topk_paged(*head, ws.data_ptr(), need, stream)
        name = "fp4idx_logits_topk_paged"
    assert rc == 0, (name, rc, L.fp4idx_strerror(rc))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


CASES = [
    # fewer than 512 rows (logits in the scratch, long-row top-k), then smaller ones
    ("verify_ctx100000", lambda: wl.config1(100_000), 2048),
    ("two_requests_20000", lambda: wl.make_logits("r2", q_per_req=[1, 1], ctx=[20000, 9000], H=32,
                                                  seed=71), 512),
    ("one_row_3000", lambda: wl.make_logits("r1", q_per_req=[1], ctx=[3000], H=16, seed=73), 64),
    # 512 rows or more (sampled threshold, kept scores in the scratch), then smaller
    ("many_rows_560", lambda: wl.make_logits("m560", q_per_req=[300, 260], ctx=[4000, 2500], H=8,
                                             seed=79), 256),
    ("verify_ctx16384", lambda: wl.config1(16384), 2048),
]


def test_noalloc_matches_the_workspace_entry_point_on_successive_calls():
    for name, make, k in CASES:
        case = make()
        say(f"[gpu] noalloc vs workspace: {name} T={case.T} out_cols={case.out_cols} k={k}")
        ai, av = _call(case, k, noalloc=False)
        bi, bv = _call(case, k, noalloc=True)
        np.testing.assert_array_equal(bi, ai)
        np.testing.assert_array_equal(bv.view(np.uint32), av.view(np.uint32))
    # and once more the first case after the others left their contents in the scratch
    name, make, k = CASES[0]
    case = make()
    say(f"[gpu] noalloc again: {name}")
    ai, av = _call(case, k, noalloc=False)
    bi, bv = _call(case, k, noalloc=True)
    np.testing.assert_array_equal(bi, ai)
    np.testing.assert_array_equal(bv.view(np.uint32), av.view(np.uint32))
