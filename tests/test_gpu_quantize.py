"""GPU parity of fp4idx_quantize_store_k against the CPU oracle.

Quantization is integer and byte work: the cache the GPU writes must equal the
oracle's byte for byte, including untouched tokens.  Keys are bf16; blocks cover
exact ties of the rounding rule, zeros and -0, saturation, and the exponent clamps.
"""
import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import check_logits, dev, say

pytestmark = pytest.mark.gpu


def _bf16(x):
    """float array -> (bf16 torch tensor on the CPU, the same values as float64)."""
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


def _keys(rng, N):
    k = rng.standard_normal((N, 128)) * 2.0 ** rng.integers(-30, 30, (N, 1))
    k[0, :32] = 0.0                                     # all-zero block
    k[0, 32:64] = -0.0
    if N > 1:                                           # exact ties at scale 1 (amax 6)
        k[1, :32] = np.resize([6.0, 5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -5.0, -0.25], 32)
        k[1, 32:64] = np.resize([7.5, 1.0, -7.0, 0.5], 32)   # saturation at 6 (amax in [4, 8))
        k[1, 64:96] = 2.0 ** -130                       # subnormal block: code clamped to 1
        k[1, 96:] = np.resize([2.0 ** 127, 2.0 ** 126, -3.0 * 2.0 ** 125], 32)  # code clamped to 254
    return k


@pytest.mark.parametrize("N,page,P", [(1, 64, 1), (37, 64, 3), (300, 128, 5), (5000, 64, 100)])
def test_quantize_store_matches_oracle(N, page, P):
    rng = np.random.default_rng(N + page)
    kt, kd = _bf16(_keys(rng, N))
    slots = rng.permutation(P * page)[:N].astype(np.int64)
    slots[5::11] = -1                                   # skipped
    if N > 3:
        slots[3] = P * page + 5                         # outside the cache: skipped
    kf0 = rng.integers(0, 256, (P, 1, page, 64), dtype=np.uint8)
    ks0 = rng.integers(0, 256, (P, 1, page, 4), dtype=np.uint8)
    want_f, want_s = orc.quantize_store(kd, slots, kf0, ks0)
    say(f"[gpu] quantize_store N={N} page={page} P={P}")
    gf, gs = dev(kf0), dev(ks0)
    fp4.quantize_store_k(kt.to("cuda"), dev(slots), gf, gs)
    torch.cuda.synchronize()
    assert np.array_equal(gf.cpu().numpy(), want_f)
    assert np.array_equal(gs.cpu().numpy(), want_s)


def test_quantized_cache_feeds_the_scorer():
    """Keys quantized on the GPU, then scored: same logits as the oracle on the cache the
    oracle quantizes."""
    rng = np.random.default_rng(5)
    ctx, page = 700, 64
    P = -(-ctx // page)
    kt, kd = _bf16(rng.standard_normal((ctx, 128)))
    perm = rng.permutation(P).astype(np.int32)
    slots = (perm[np.arange(ctx) // page].astype(np.int64) * page + np.arange(ctx) % page)
    case = wl.make_logits("qcache", q_per_req=[4], ctx=[ctx], H=32, seed=6,
                          row_lens=[ctx, ctx - 1, 300, 1])
    case.block_table[0, :P] = perm
    zf = np.zeros((P, 1, page, 64), np.uint8)
    zs = np.full((P, 1, page, 4), 127, np.uint8)
    case.k_fp4, case.k_scale = orc.quantize_store(kd, slots, zf, zs)
    gf, gs = dev(zf), dev(zs)
    say("[gpu] quantize_store + logits")
    fp4.quantize_store_k(kt.to("cuda"), dev(slots), gf, gs)
    got = fp4.logits_paged(dev(case.q_fp4), dev(case.q_scale), dev(case.w), gf, gs,
                           dev(case.block_table), dev(case.cu_seqlens_q), dev(case.row_lens),
                           out_cols=case.out_cols)
    torch.cuda.synchronize()
    assert np.array_equal(gf.cpu().numpy(), case.k_fp4)
    ref, tb, inexact = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                        case.k_scale, case.block_table, case.cu_seqlens_q,
                                        case.row_lens, case.page_size, case.out_cols,
                                        want_tolbase=True)
    assert inexact == 0
    check_logits(got.cpu().numpy(), ref, tb)


@pytest.mark.parametrize("key_rs,kp_extra,ksp_extra,key_off", [
    (128, 0, 0, 0),      # contiguous: 16-byte key loads, 4-byte nibble stores
    (132, 6, 3, 2),      # key rows 4-byte aligned only, odd page strides: the narrow paths
    (130, 2, 1, 0),      # key row stride 260 bytes, page strides not multiples of 4
])
def test_quantize_store_strided_through_the_c_abi(key_rs, kp_extra, ksp_extra, key_off):
    """fp4idx_quantize_store_k with key rows and cache pages padded: every written byte
    equals the oracle's, the padding between rows and pages is left as it was."""
    from sparse_attention_fp4_amd._lib import lib
    rng = np.random.default_rng(key_rs + kp_extra)
    N, page, P = 200, 64, 5
    k = _keys(rng, N)
    kt, kd = _bf16(k)
    slots = rng.permutation(P * page)[:N].astype(np.int64)
    slots[7::13] = -1
    # keys: [key_off + N * key_rs] bf16, row n at key_off + n * key_rs
    kb = torch.zeros(key_off + N * key_rs + 8, dtype=torch.bfloat16)
    kb[key_off:key_off + N * key_rs].view(N, key_rs)[:, :128] = kt
    kp, ksp = page * 64 + kp_extra, page * 4 + ksp_extra
    kf0 = rng.integers(0, 256, (P, 1, page, 64), dtype=np.uint8)
    ks0 = rng.integers(0, 256, (P, 1, page, 4), dtype=np.uint8)
    fbuf = rng.integers(0, 256, P * kp, dtype=np.uint8)       # pages padded with noise
    sbuf = rng.integers(0, 256, P * ksp, dtype=np.uint8)
    for p_ in range(P):
        fbuf[p_ * kp:p_ * kp + page * 64] = kf0[p_].reshape(-1)
        sbuf[p_ * ksp:p_ * ksp + page * 4] = ks0[p_].reshape(-1)
    want_f, want_s = orc.quantize_store(kd, slots, kf0, ks0)
    gk, gsl, gf, gs = kb.to("cuda"), dev(slots), dev(fbuf), dev(sbuf)
    say(f"[gpu] quantize_store strided key_rs={key_rs} kp={kp} ksp={ksp} key_off={key_off}")
    rc = lib().fp4idx_quantize_store_k(gk.data_ptr() + 2 * key_off, key_rs, gsl.data_ptr(), N,
                                       gf.data_ptr(), kp, gs.data_ptr(), ksp, page, P,
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    gotf, gots = gf.cpu().numpy(), gs.cpu().numpy()
    for p_ in range(P):
        assert np.array_equal(gotf[p_ * kp:p_ * kp + page * 64], want_f[p_].reshape(-1)), p_
        assert np.array_equal(gotf[p_ * kp + page * 64:(p_ + 1) * kp], fbuf[p_ * kp + page * 64:(p_ + 1) * kp])
        assert np.array_equal(gots[p_ * ksp:p_ * ksp + page * 4], want_s[p_].reshape(-1)), p_
        assert np.array_equal(gots[p_ * ksp + page * 4:(p_ + 1) * ksp], sbuf[p_ * ksp + page * 4:(p_ + 1) * ksp])
