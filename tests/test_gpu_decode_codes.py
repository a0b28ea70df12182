"""Every stored code through the GPU scorer, compared bit for bit with the oracle.

"[DSv4.1] Speed up the FP4 indexer scorer..." (Modifications, Accuracy Tests): the
scorer must decode every E2M1 nibble and every E8M0 scale code exactly.  "M3 FP4
Indexer" README (FP4 和 scale layout): NVFP4 block scales are float8_e4m3fn, with no
restriction on their range.

One-hot operands expose single products: a query whose only nonzero element is element
d (nibble n, scale code c) against a key of +-1 values (or the other way round) gives
the dot E2M1(n) * scale_q * (+-1) * scale_k, one exact product.  Through the logits
(H = 1, weight 1) the value seen is ReLU(dot); a key of -1 values shows the negative
side.  Through the block scores (one valid key per batch item) the value seen is the dot
itself.  Where the exact product is 0 or a normal fp32 number the GPU must return the
oracle's value bit for bit; products outside that range (E8M0 only: overflow to inf or
fp32 subnormals) are reported, not asserted.

MXFP4 covers: all 16 nibbles x E8M0 codes 1..254 on the query side and on the key side,
each against every key (query) scale code 1..254 of the other side.  NVFP4 covers: all
16 nibbles x the 254 non-NaN E4M3 codes (both signs, the subnormals, 0x00, 0x80 and
+-448) on each side, against every non-NaN code of the other side.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import gpu_block_scores, gpu_logits, oracle_block_scores, oracle_logits, say

pytestmark = pytest.mark.gpu

E8M0 = np.arange(1, 255, dtype=np.uint8)                                 # stored range
E4M3 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)  # non-NaN codes
ONE = {wl.MXFP4: 127, wl.NVFP4: 0x38}                                    # scale 1.0
PLUS1, MINUS1 = 0x22, 0xAA                                               # bytes of +1 / -1 pairs


def _codes(fmt):
    return E8M0 if fmt == wl.MXFP4 else E4M3


def _one_hot(n_vec, fmt, codes, nibbles, seed):
    """n_vec packed vectors: vector i has nibble nibbles[i] at element d_i = (7i + 3) % 128
    and zeros elsewhere; the scale of d_i's group is codes[i], the other groups get
    random codes of the format's stored range (their elements are zero)."""
    G = wl.groups(fmt)
    S = 128 // G
    rng = np.random.default_rng(seed)
    packed = np.zeros((n_vec, 64), np.uint8)
    pool = _codes(fmt)
    scales = pool[rng.integers(0, pool.size, size=(n_vec, G))].astype(np.uint8)
    d = (7 * np.arange(n_vec) + 3) % 128
    i = np.arange(n_vec)
    nib = np.asarray(nibbles, np.uint8)
    packed[i, d // 2] = np.where(d % 2 == 0, nib, nib << 4).astype(np.uint8)
    scales[i, d // S] = codes
    return packed, scales


def _signed_ones(n_vec, fmt, codes):
    """Vector 2j + s: every element +1 (s = 0) or -1 (s = 1), every scale codes[j]."""
    G = wl.groups(fmt)
    packed = np.empty((n_vec, 64), np.uint8)
    packed[0::2] = PLUS1
    packed[1::2] = MINUS1
    scales = np.repeat(np.asarray(codes, np.uint8), 2)[:, None].repeat(G, axis=1)
    return packed, scales


def _exact_mask(exact):
    """Where the result must be matched bit for bit: the exact value (float64, computed
    from the oracle's decoders) is zero or a normal fp32 number."""
    a = np.abs(exact)
    return (a == 0) | ((a >= 2.0 ** -126) & (a < 2.0 ** 128))


def _logits_case(name, fmt, q_packed, q_scales, k_packed, k_scales, seed):
    T, P_keys = q_packed.shape[0], k_packed.shape[0]
    case = wl.make_logits(name, fmt=fmt, q_per_req=[T], ctx=[P_keys], H=1, seed=seed)
    pages = case.num_pages
    kf = np.zeros((pages * 64, 64), np.uint8)
    ks = np.full((pages * 64, wl.groups(fmt)), ONE[fmt], np.uint8)
    kf[:P_keys] = k_packed
    ks[:P_keys] = k_scales
    # logical key s sits on physical page block_table[0][s // 64]
    phys = case.block_table[0, np.arange(pages)]
    case.k_fp4 = np.zeros((pages, 1, 64, 64), np.uint8)
    case.k_scale = np.zeros((pages, 1, 64, wl.groups(fmt)), np.uint8)
    case.k_fp4[phys, 0] = kf.reshape(pages, 64, 64)
    case.k_scale[phys, 0] = ks.reshape(pages, 64, -1)
    case.q_fp4 = q_packed[:, None, :].copy()
    case.q_scale = q_scales[:, None, :].copy()
    case.w = np.ones((T, 1), np.float32)
    return case


def _compare(tag, got, ref, exact):
    must = _exact_mask(exact)
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    bad = must & (gb != rb)
    say(f"    {tag}: {int(must.sum())} in-range values, {int(bad.sum())} differ; "
        f"out of range: {int((~must).sum())}, equal there: {int(((~must) & (gb == rb)).sum())}")
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{tag}: first difference at {tuple(i)}: got {got[tuple(i)]!r} "
                             f"oracle {ref[tuple(i)]!r}")


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4], ids=["mxfp4", "nvfp4"])
@pytest.mark.parametrize("side", ["query", "key"])
def test_logits_decode_every_code(fmt, side):
    codes = _codes(fmt)
    nc = codes.size
    # 16 nibbles x every code on the swept side; +-1 vectors at every code on the other
    nib = np.repeat(np.arange(16, dtype=np.uint8), nc)
    cod = np.tile(codes, 16)
    sweep_p, sweep_s = _one_hot(16 * nc, fmt, cod, nib, seed=41 + fmt)
    ones_p, ones_s = _signed_ones(2 * nc, fmt, codes)
    if side == "query":
        case = _logits_case(f"codes_q_{fmt}", fmt, sweep_p, sweep_s, ones_p, ones_s, seed=43)
    else:
        case = _logits_case(f"codes_k_{fmt}", fmt, ones_p, ones_s, sweep_p, sweep_s, seed=47)
    got = gpu_logits(case)
    ref, _, inexact = oracle_logits(case)
    assert inexact == 0
    assert not np.any(ref == -np.inf) and not np.any(got == -np.inf)
    Qd = orc.dequant(fmt, case.q_fp4[:, 0], case.q_scale[:, 0])
    n_keys = case.out_cols
    Kl = orc.dequant(fmt, case.k_fp4[case.block_table[0, :case.num_pages], 0],
                     case.k_scale[case.block_table[0, :case.num_pages], 0]).reshape(-1, 128)[:n_keys]
    exact = np.maximum(Qd @ Kl.T, 0.0)   # one nonzero product per pair: exact in double
    _compare(f"logits, {side} codes swept", got, ref, exact)


def _block_case(name, fmt, q_packed, q_scales, k_packed, k_scales, Hq, seed):
    """Batch item b: one key (row b of k_packed) on its own 128-token page, Tq / B
    queries of Hq heads each, non-causal; scores[h, 0, q] is the dot of query q, head h
    with its item's key."""
    B = k_packed.shape[0]
    Tq = q_packed.shape[0] // Hq
    assert Tq % B == 0
    per = Tq // B
    case = wl.make_block(name, fmt=fmt, q_lens=[per] * B, k_lens=[1] * B, Hq=Hq, Hkv=1,
                         seed=seed, causal=False)
    G = wl.groups(fmt)
    case.k_fp4[:] = 0
    case.k_scale[:] = ONE[fmt]
    phys = case.kv_indices[case.cu_page_offsets[:-1]]
    case.k_fp4[phys, 0, 0] = k_packed
    case.k_scale[phys, 0, 0] = k_scales
    case.q_fp4 = q_packed.reshape(Tq, Hq, 64).copy()
    case.q_scale = q_scales.reshape(Tq, Hq, G).copy()
    return case


def _block_exact(case):
    """[Hq, 1, Tq] float64: each query head's dot with its item's single key."""
    Qd = orc.dequant(case.fmt, case.q_fp4, case.q_scale)              # [Tq, Hq, 128]
    item = np.searchsorted(case.cu_seqlens_q, np.arange(case.Tq), side="right") - 1
    phys = case.kv_indices[case.cu_page_offsets[item]]
    Kd = orc.dequant(case.fmt, case.k_fp4[phys, 0, 0], case.k_scale[phys, 0, 0])  # [Tq, 128]
    return np.einsum("qhd,qd->hq", Qd, Kd)[:, None, :]


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4], ids=["mxfp4", "nvfp4"])
def test_block_scores_decode_every_query_code(fmt):
    """Item b (2 per key code: +1 and -1 keys); its query has 16 heads, head h holding
    nibble h at the item's query code, so every (nibble, code) pair appears on the query
    side twice.  MXFP4 pairs query code 255 - c_k with key code c_k (products stay at
    2^1 * E2M1); NVFP4 takes query codes (37 b) mod 254 of the code list."""
    codes = _codes(fmt)
    nc = codes.size
    kp, ks = _signed_ones(2 * nc, fmt, codes)
    B = 2 * nc
    b = np.arange(B)
    if fmt == wl.MXFP4:
        qcode = np.clip(255 - codes[b // 2].astype(np.int64), 1, 254).astype(np.uint8)
    else:
        qcode = codes[(37 * b) % nc]
    nib = np.tile(np.arange(16, dtype=np.uint8), B)
    qp, qs = _one_hot(B * 16, fmt, np.repeat(qcode, 16), nib, seed=53 + fmt)
    case = _block_case(f"bcodes_q_{fmt}", fmt, qp, qs, kp, ks, Hq=16, seed=59)
    got = gpu_block_scores(case)
    ref, _, inexact = oracle_block_scores(case)
    assert inexact == 0
    _compare("block scores, query codes swept", got, ref, _block_exact(case))


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.NVFP4], ids=["mxfp4", "nvfp4"])
def test_block_scores_decode_every_key_code(fmt):
    """Item b holds one one-hot key (nibble b // ncodes at code b % ncodes); its query
    has two heads, +1 and -1 values, at code 255 - c_k (MXFP4) or code (37 b) mod 254 of
    the list (NVFP4)."""
    codes = _codes(fmt)
    nc = codes.size
    B = 16 * nc
    b = np.arange(B)
    kcode = codes[b % nc]
    kp, ks = _one_hot(B, fmt, kcode, (b // nc).astype(np.uint8), seed=61 + fmt)
    if fmt == wl.MXFP4:
        qcode = np.clip(255 - kcode.astype(np.int64), 1, 254).astype(np.uint8)
    else:
        qcode = codes[(37 * b) % nc]
    G = wl.groups(fmt)
    qp = np.empty((B, 2, 64), np.uint8)
    qp[:, 0] = PLUS1
    qp[:, 1] = MINUS1
    qs = np.repeat(qcode[:, None], 2 * G, axis=1).reshape(B, 2, G)
    case = _block_case(f"bcodes_k_{fmt}", fmt, qp.reshape(B * 2, 64), qs.reshape(B * 2, G),
                       kp, ks, Hq=2, seed=67)
    got = gpu_block_scores(case)
    ref, _, inexact = oracle_block_scores(case)
    assert inexact == 0
    _compare("block scores, key codes swept", got, ref, _block_exact(case))
