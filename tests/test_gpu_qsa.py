"""GPU parity of the sparse attention over selected tokens (vLLM qsa_fp8 API page).

Slot pass: integer work, equal to the oracle's slots bit for bit.

Decode: compared element by element with the oracle's double-precision result on the
same seeded inputs.  The kernel computes as the page does: exact bf16 x e4m3 products
summed in fp32, probabilities rounded to fp16 for the product with V (fp32
normalizer), the normalized output rounded to bf16, multiplied by sigmoid(gate) and
rounded to bf16 again.  Bound derived from that arithmetic, with tolbase =
|output_scale| * sum_j a_j |V_j[d]| * sigmoid(gate) (the oracle's size of the summed
terms):
  * fp16 rounding of each probability: at most 2^-11 of tolbase;
  * fp32 score sums over 128 products (<= 128 * 2^-24 of the score's magnitude sum) and
    the exp2 / rescale roundings: below 2^-13 of tolbase for these inputs;
  * the two bf16 roundings of the output: bf16 keeps 8 significant bits, so each is at
    most 2^-8 relative, 2^-7 of |out| together (plus 2^-16 of tolbase).
So |gpu - oracle| <= 2^-7 |oracle| + 2^-9.8 tolbase, element by element.
"""
import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import say

pytestmark = pytest.mark.gpu


def _bits_to_float(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _upload(case, separate=False, q_pad=0):
    """Device tensors of a case.  separate: K and V in two caches with equal block and
    token strides but different head strides (D for K, 2D for V); q_pad: extra elements
    between q / gate / out rows."""
    D, Hkv = case.D, case.Hkv
    if separate:
        k = torch.from_numpy(np.ascontiguousarray(case.k_cache)).cuda()
        v = torch.from_numpy(np.ascontiguousarray(case.v_cache)).cuda()
        P, page = k.shape[:2]
        kbuf = torch.zeros((P, page, 2 * Hkv, D), dtype=torch.uint8, device="cuda")
        vbuf = torch.zeros_like(kbuf)
        kbuf[:, :, :Hkv] = k
        vbuf[:, :, ::2] = v
        kc, vc = kbuf[:, :, :Hkv], vbuf[:, :, ::2]
        assert kc.stride()[:2] == vc.stride()[:2] and kc.stride(2) != vc.stride(2)
    else:
        kv = torch.from_numpy(case.kv).cuda()
        kc = kv.permute(0, 2, 1, 3)[..., :D]
        vc = kv.permute(0, 2, 1, 3)[..., D:]

    def padded(bits):
        rows, H, _ = bits.shape
        if not q_pad:
            return _bf16_dev(bits)
        buf = torch.zeros((rows, H * D + q_pad), dtype=torch.bfloat16, device="cuda")
        buf[:, :H * D] = _bf16_dev(bits).reshape(rows, H * D)
        return buf[:, :H * D].view(rows, H, D)

    q = padded(case.q)
    gate = padded(case.gate)
    out = padded(np.full(case.q.shape, 0x7FC0, np.uint16))   # NaN: every element is written
    return dict(k=kc, v=vc, q=q, gate=gate, out=out,
                ind=torch.from_numpy(case.indices).cuda(),
                bt=torch.from_numpy(case.block_table).cuda(),
                t2r=torch.from_numpy(case.token_to_req).cuda())


def _run_gpu(case, d, slot_cols=None):
    say(f"[gpu] qsa {case.name} rows={case.rows} Hq={case.Hq} Hkv={case.Hkv} "
        f"page={case.page_size} topk={case.topk} blocks={case.num_cache_blocks}")
    slots = torch.full((case.rows, slot_cols or case.topk), 12345, dtype=torch.int32,
                       device="cuda")
    fp4.qsa_sparse_paged_decode(d["q"], d["k"], d["v"], d["ind"], d["bt"], d["t2r"], d["out"],
                                d["gate"], case.softmax_scale, case.output_scale, slots=slots)
    torch.cuda.synchronize()
    got = d["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    return slots.cpu().numpy(), got


def _check(case, slots_gpu, out_bits, rows=None):
    slot_cols = slots_gpu.shape[1]
    so = orc.qsa_slots(case.indices, case.block_table, case.token_to_req, case.num_cache_blocks,
                       case.page_size, slot_cols)
    np.testing.assert_array_equal(slots_gpu, so)
    want, tb = orc.qsa_decode(case.q, case.k_cache, case.v_cache, so, case.indices,
                              orc.qsa_offset_bits(case.page_size), case.softmax_scale,
                              case.output_scale, case.gate, rows=rows, want_tolbase=True)
    got = _bits_to_float(out_bits if rows is None else out_bits[np.asarray(rows)])
    assert np.isfinite(got).all()
    err = np.abs(got - want)
    tol = 2.0 ** -7 * np.abs(want) + 2.0 ** -9.8 * tb
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements off, first {tuple(i)}: gpu {got[tuple(i)]} "
                             f"oracle {want[tuple(i)]} tol {tol[tuple(i)]}")
    # rows with nothing selected are exactly zero
    n = np.clip(case.indices[:, -1], 0, case.topk)
    empty = [r for r in range(case.rows) if not (so[r, :n[r]] >= 0).any()]
    if rows is None and empty:
        assert not got[empty].any()
    return err, tol


def _case(name, **kw):
    return wl.make_qsa(name, **kw)


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (16, 1), (48, 16), (12, 4), (8, 8), (2, 1)])
def test_decode_group_sizes(Hq, Hkv):
    case = _case(f"groups_{Hq}_{Hkv}", ctx=[300, 1000, 77, 4096, 2000, 129], Hq=Hq, Hkv=Hkv,
                 topk=256, page=64, seed=Hq * 100 + Hkv)
    slots, out = _run_gpu(case, _upload(case))
    _check(case, slots, out)


@pytest.mark.parametrize("page", [16, 64, 128, 48, 1])
def test_decode_page_sizes(page):
    case = _case(f"page_{page}", ctx=[513, 2000, 40, 999], Hq=32, Hkv=4, topk=320, page=page,
                 seed=700 + page, extra_pages=3)
    slots, out = _run_gpu(case, _upload(case), slot_cols=333)
    _check(case, slots, out)


def test_decode_counts_at_chunk_edges_and_masked_entries():
    """Valid counts 0, 1, 31, 32, 33, 63, 64, 65, topk, negative and above topk; -1 entries,
    duplicates, tokens past the table width, pages outside the cache and bad requests."""
    case = _case("edges", ctx=[5000] * 12, Hq=32, Hkv=4, topk=96, page=64, seed=4242,
                 drop_frac=0.1)
    ind = case.indices
    counts = [0, 1, 31, 32, 33, 63, 64, 65, 96, -5, 500, 96]
    for r, c in enumerate(counts):
        ind[r, -1] = c
    ind[11, 5] = ind[11, 6]                    # duplicate
    ind[11, 7] = 10 ** 6                       # past the table width
    ind[10, 3] = ind[10, 4] = 4990             # duplicates near the end
    bt = case.block_table
    bt[3, 1] = -1                              # a hole in a request's table
    bt[4, 0] = case.num_cache_blocks + 7       # a page outside the cache
    case.token_to_req[5] = 12                  # a request that does not exist
    case.token_to_req[6] = -2
    slots, out = _run_gpu(case, _upload(case))
    _check(case, slots, out)


def test_decode_all_finite_codes_and_output_scale():
    """K and V over every finite e4m3fn code (subnormals, zeros, +-448) with a small
    softmax scale, a negative output scale and wide gates."""
    case = _case("codes", ctx=[700, 3000, 256], Hq=32, Hkv=4, topk=512, page=64, seed=99,
                 k_exp=(0, 15), gate_exp=(-6, 4), softmax_scale=2.0 ** -9, output_scale=-0.37)
    slots, out = _run_gpu(case, _upload(case))
    _check(case, slots, out)


def test_decode_separate_caches_and_strided_rows():
    case = _case("separate", ctx=[900, 4000, 1500, 64], Hq=24, Hkv=3, topk=384, page=32,
                 seed=1234)
    slots, out = _run_gpu(case, _upload(case, separate=True, q_pad=24))
    _check(case, slots, out)


def test_decode_indexer_topk_output_feeds_the_slot_pass():
    """The indexer's own top-k output (increasing token order, -1 padded) with its count
    appended is a valid selection: decode over it equals the oracle."""
    case = _case("from_topk", ctx=[3000, 700, 2048], Hq=32, Hkv=4, topk=1024, page=64, seed=5)
    rng = np.random.default_rng(6)
    rows = case.rows
    scores = rng.standard_normal((rows, 3000)).astype(np.float32)
    lens = np.array([case.meta["ctx"][int(b)] for b in case.token_to_req], np.int32)
    for r in range(rows):
        scores[r, lens[r]:] = -np.inf
    idx, _ = fp4.topk(torch.from_numpy(scores).cuda(), case.topk,
                      torch.from_numpy(lens).cuda(), want_vals=False)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    ind = np.full((rows, case.topk + 1), -1, np.int32)
    ind[:, :case.topk] = idx
    ind[:, -1] = (idx >= 0).sum(axis=1)
    case.indices = ind
    slots, out = _run_gpu(case, _upload(case))
    _check(case, slots, out)


def test_decode_full_size_sampled_rows():
    """The benchmark's workload (128 rows x top-2048, Hq=32, Hkv=4, contexts
    U[8192, 32768]) in its launch configuration; 8 sampled rows against the oracle."""
    case = wl.qsa_decode_case()
    slots, out = _run_gpu(case, _upload(case))
    rng = np.random.default_rng(1051)
    rows = sorted(rng.choice(case.rows, 8, replace=False).tolist()) + [case.rows - 1]
    _check(case, slots, out, rows=rows)
