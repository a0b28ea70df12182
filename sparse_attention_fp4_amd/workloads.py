"""Seeded synthetic inputs for the FP4 indexer workloads.

This module only draws random codes and builds page tables and length metadata with
numpy.  It decodes nothing and computes no score: both the GPU library's tests and the
CPU oracle take their inputs from here, and nothing else is shared between them.

Value distributions follow the pages' workloads:
  * E2M1 nibbles uniform over the 16 codes (so every byte is uniform over 0..255);
  * E8M0 scale codes uniform in a stated range (123..131 or 120..134);
  * E4M3 scale codes 2^e * (1 + m/8) with e uniform in [-4, 4] and m uniform in
    [0, 7], i.e. code ((e + 7) << 3) | m;
  * head weights w = k/64 with k uniform in [-64, 64] (exact in fp32);
  * physical pages in a random permutation, addressed through a block table
    ("[DSv4.1] Speed up the FP4 indexer scorer..." bench: keys on shuffled 64-token
    pages; "M3 FP4 Indexer" README, 输入 shape 和类型: kv_indices maps logical pages).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MXFP4 = 0
NVFP4 = 1


def groups(fmt: int) -> int:
    return 4 if fmt == MXFP4 else 8


@dataclass
class LogitsCase:
    """Inputs of one weighted-ReLU logits call (host arrays)."""
    name: str
    fmt: int
    q_fp4: np.ndarray        # [T, H, 64] uint8
    q_scale: np.ndarray      # [T, H, G] uint8
    w: np.ndarray            # [T, H] float32
    k_fp4: np.ndarray        # [P, Hkv, page, 64] uint8
    k_scale: np.ndarray      # [P, Hkv, page, G] uint8
    block_table: np.ndarray  # [B, W] int32, -1 padded
    cu_seqlens_q: np.ndarray  # [B+1] int32
    row_lens: np.ndarray     # [T] int32
    page_size: int
    out_cols: int
    topk: int = 2048
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q_fp4.shape[0]

    @property
    def H(self):
        return self.q_fp4.shape[1]

    @property
    def Hkv(self):
        return self.k_fp4.shape[1]

    @property
    def B(self):
        return self.block_table.shape[0]

    @property
    def num_pages(self):
        return self.k_fp4.shape[0]

    def visible_pairs(self) -> int:
        return int(np.minimum(self.row_lens, self.out_cols).clip(min=0).sum())

    def unique_keys(self) -> int:
        """Keys of each request read at least once (max row_len per request)."""
        n = 0
        for b in range(self.B):
            lo, hi = int(self.cu_seqlens_q[b]), int(self.cu_seqlens_q[b + 1])
            if hi > lo:
                n += int(min(self.row_lens[lo:hi].max(), self.out_cols))
        return n


@dataclass
class BlockCase:
    """Inputs of one per-head block-max call (host arrays)."""
    name: str
    fmt: int
    q_fp4: np.ndarray          # [Tq, Hq, 64] uint8
    q_scale: np.ndarray        # [Tq, Hq, G] uint8
    k_fp4: np.ndarray          # [P, Hkv, 128, 64] uint8
    k_scale: np.ndarray        # [P, Hkv, 128, G] uint8
    cu_seqlens_q: np.ndarray   # [B+1] int32
    cu_seqlens_k: np.ndarray   # [B+1] int32
    cu_page_offsets: np.ndarray  # [B+1] int32
    kv_indices: np.ndarray     # [P] int32
    qo_offset: Optional[np.ndarray]  # [B] int32 or None
    max_seqlen_q: int
    max_seqlen_k: int
    causal: bool
    meta: dict = field(default_factory=dict)

    @property
    def Tq(self):
        return self.q_fp4.shape[0]

    @property
    def Hq(self):
        return self.q_fp4.shape[1]

    @property
    def Hkv(self):
        return self.k_fp4.shape[1]

    @property
    def B(self):
        return self.cu_seqlens_q.size - 1

    @property
    def ktiles(self):
        return (self.max_seqlen_k + 127) // 128

    def visible_pairs(self) -> int:
        """Visible (query, key) pairs summed over the batch (no head factor)."""
        n = 0
        for b in range(self.B):
            ql = int(self.cu_seqlens_q[b + 1] - self.cu_seqlens_q[b])
            kl = int(self.cu_seqlens_k[b + 1] - self.cu_seqlens_k[b])
            if not self.causal:
                n += ql * kl
                continue
            off = int(self.qo_offset[b]) if self.qo_offset is not None else kl - ql
            q = np.arange(ql, dtype=np.int64)
            n += int(np.clip(q + off + 1, 0, kl).sum())
        return n


def _codes(rng, shape):
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def _scales(rng, fmt, shape, e8_lo=123, e8_hi=131):
    if fmt == MXFP4:
        return rng.integers(e8_lo, e8_hi + 1, size=shape, dtype=np.uint8)
    e = rng.integers(-4, 5, size=shape)
    m = rng.integers(0, 8, size=shape)
    return (((e + 7) << 3) | m).astype(np.uint8)


def _weights(rng, shape):
    return (rng.integers(-64, 65, size=shape).astype(np.float32) / np.float32(64.0))


def make_logits(name, *, fmt=MXFP4, q_per_req, ctx, H, Hkv=1, page=64, seed=0,
                e8_lo=123, e8_hi=131, row_lens=None, out_cols=None, table_width=None,
                topk=2048) -> LogitsCase:
    """General decode/prefill logits case.

    q_per_req[b] query rows for request b, which holds ctx[b] keys.  Unless row_lens is
    given, every row of request b sees all ctx[b] keys.  Pages of all requests are
    disjoint and globally shuffled; block_table rows are -1 padded.
    """
    rng = np.random.default_rng(seed)
    q_per_req = [int(x) for x in q_per_req]
    ctx = [int(x) for x in ctx]
    B = len(ctx)
    T = sum(q_per_req)
    G = groups(fmt)
    npg = [max(1, -(-c // page)) for c in ctx]
    P = sum(npg)
    W = table_width if table_width is not None else max(npg)
    if out_cols is None:
        out_cols = max(ctx)
    # tensor order: q_fp4, q_scale, w, k_fp4, k_scale, tables
    q_fp4 = _codes(rng, (T, H, 64))
    q_scale = _scales(rng, fmt, (T, H, G), e8_lo, e8_hi)
    w = _weights(rng, (T, H))
    k_fp4 = _codes(rng, (P, Hkv, page, 64))
    k_scale = _scales(rng, fmt, (P, Hkv, page, G), e8_lo, e8_hi)
    perm = rng.permutation(P).astype(np.int32)
    block_table = np.full((B, W), -1, np.int32)
    o = 0
    for b in range(B):
        block_table[b, :npg[b]] = perm[o:o + npg[b]]
        o += npg[b]
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(q_per_req)
    if row_lens is None:
        row_lens = np.concatenate([np.full(q_per_req[b], ctx[b], np.int32) for b in range(B)])
    row_lens = np.asarray(row_lens, np.int32)
    return LogitsCase(name, fmt, q_fp4, q_scale, w, k_fp4, k_scale, block_table, cu, row_lens,
                      page, int(out_cols), topk, {"ctx": ctx, "seed": seed})


def verify_rows_case(ctx, *, seed, name=None, H=32, rows=4, page=64, fmt=MXFP4):
    """One request, `rows` verify rows that see ctx, ctx-1, ..., ctx-rows+1 keys."""
    lens = np.array([ctx - i for i in range(rows)], np.int32)
    return make_logits(name or f"verify_ctx{ctx}", fmt=fmt, q_per_req=[rows], ctx=[ctx], H=H,
                       page=page, seed=seed, row_lens=lens, out_cols=ctx)


def config0(seed=1000):
    """MXFP4 decode scorer, 1 request, 4 verify rows that see 2048 - 0..3 keys, H=32,
    page 64, logits [4, 2048]."""
    return verify_rows_case(2048, seed=seed, name="decode_ctx2048_h32")


def config1(ctx=100_000, seed=1010):
    """As config0 at context 16384 / 100000 / 400000, followed by top-2048."""
    return verify_rows_case(ctx, seed=seed, name=f"decode_ctx{ctx}_h32")


def config2(seed=1020):
    """64 requests x 1 row, H=64, contexts uniform in [4096, 131072], E8M0 120..134,
    block table [64, 2048], logits [64, 131072], top-2048."""
    rng = np.random.default_rng(seed + 5)
    ctx = rng.integers(4096, 131072 + 1, size=64).tolist()
    return make_logits("batched_decode_b64_h64", q_per_req=[1] * 64, ctx=ctx, H=64, seed=seed,
                       e8_lo=120, e8_hi=134, out_cols=131072, table_width=2048)


def config4(seed=1040, T=32768):
    """One request, T query tokens x T keys, H=64, causal rows (row t sees t+1 keys)."""
    lens = np.arange(1, T + 1, dtype=np.int32)
    return make_logits(f"prefill_causal_{T}_h64", q_per_req=[T], ctx=[T], H=64, seed=seed,
                       row_lens=lens, out_cols=T)


def make_block(name, *, fmt, q_lens, k_lens, Hq, Hkv, seed, causal=True, qo_offset=None,
               e8_lo=123, e8_hi=131, extra_pages=0) -> BlockCase:
    """Varlen block-score case with 128-token pages in a random permutation."""
    rng = np.random.default_rng(seed)
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    B = len(q_lens)
    G = groups(fmt)
    Tq = sum(q_lens)
    npg = [-(-k // 128) for k in k_lens]
    P = sum(npg) + extra_pages
    q_fp4 = _codes(rng, (Tq, Hq, 64))
    q_scale = _scales(rng, fmt, (Tq, Hq, G), e8_lo, e8_hi)
    k_fp4 = _codes(rng, (P, Hkv, 128, 64))
    k_scale = _scales(rng, fmt, (P, Hkv, 128, G), e8_lo, e8_hi)
    perm = rng.permutation(P).astype(np.int32)
    kv_indices = perm[:sum(npg)].copy()
    cu_q = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    cu_k = np.zeros(B + 1, np.int32)
    cu_k[1:] = np.cumsum(k_lens)
    cu_p = np.zeros(B + 1, np.int32)
    cu_p[1:] = np.cumsum(npg)
    qo = None if qo_offset is None else np.asarray(qo_offset, np.int32)
    return BlockCase(name, fmt, q_fp4, q_scale, k_fp4, k_scale, cu_q, cu_k, cu_p, kv_indices, qo,
                     max(q_lens), max(k_lens), causal, {"seed": seed})


def config3(seed=1030):
    """NVFP4 block-score prefill: B=8, q_len U[128,2048], k_len = q_len + U[0,8192],
    Hq=32, Hkv=4, causal, no qo_offset."""
    rng = np.random.default_rng(seed + 5)
    q_lens = rng.integers(128, 2048 + 1, size=8)
    k_lens = q_lens + rng.integers(0, 8192 + 1, size=8)
    return make_block("nvfp4_block_prefill_b8", fmt=NVFP4, q_lens=q_lens, k_lens=k_lens, Hq=32,
                      Hkv=4, seed=seed, causal=True)


# ---------------------------------------------------------------------------------------
# Sparse paged attention over the selected tokens (vLLM qsa_fp8 API page): an fp8 e4m3fn
# K/V cache, bf16 queries and output gates, and per-row lists of selected logical tokens.
# ---------------------------------------------------------------------------------------

@dataclass
class QsaCase:
    """Inputs of one sparse decode over selected tokens (host arrays)."""
    name: str
    kv: np.ndarray             # [blocks, Hkv, page, 2D] uint8: per token and head, D K codes
                               # then D V codes (one combined cache)
    block_table: np.ndarray    # [R, W] int32, -1 padded
    token_to_req: np.ndarray   # [rows] int32
    indices: np.ndarray        # [rows, topk + 1] int32: selected logical tokens, -1 padded,
                               # the valid count in the last column
    q: np.ndarray              # [rows, Hq, D] uint16 bf16 bit patterns
    gate: np.ndarray           # [rows, Hq, D] uint16 bf16 bit patterns
    page_size: int
    softmax_scale: float
    output_scale: float
    meta: dict = field(default_factory=dict)

    @property
    def rows(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def Hkv(self):
        return self.kv.shape[1]

    @property
    def topk(self):
        return self.indices.shape[1] - 1

    @property
    def num_cache_blocks(self):
        return self.kv.shape[0]

    @property
    def k_cache(self):
        """[blocks, page, Hkv, D] view of the K codes."""
        return self.kv.transpose(0, 2, 1, 3)[..., :self.D]

    @property
    def v_cache(self):
        return self.kv.transpose(0, 2, 1, 3)[..., self.D:]

    def selected(self) -> int:
        """Selected (row, token) pairs with a valid entry before the count."""
        n = 0
        for r in range(self.rows):
            c = int(np.clip(self.indices[r, -1], 0, self.topk))
            n += int((self.indices[r, :c] >= 0).sum())
        return n


def e4m3_codes(rng, shape, exp_lo=4, exp_hi=7):
    """Uniform e4m3fn codes (sign << 7 | exponent field << 3 | mantissa) with exponent
    field in [exp_lo, exp_hi] (values 2^(e-7) * (1 + m/8); field 0 gives the subnormals
    m/8 * 2^-6), sign uniform, the NaN codes 0x7F / 0xFF never drawn."""
    size = int(np.prod(shape))
    if (exp_lo, exp_hi) == (4, 7):
        # fields 4..7 are 0b01xx: a random byte with bit 6 cleared and bit 5 set is a
        # uniform draw over these 64 codes
        words = rng.integers(0, 2**64 - 1, size=-(-size // 8), dtype=np.uint64, endpoint=True)
        raw = words.view(np.uint8)[:size]
        np.bitwise_and(raw, 0x9F, out=raw)
        np.bitwise_or(raw, 0x20, out=raw)
        return raw.reshape(shape)
    allowed = np.array([(s << 7) | (e << 3) | m for s in (0, 1)
                        for e in range(exp_lo, exp_hi + 1) for m in range(8)
                        if not (e == 15 and m == 7)], np.uint8)
    return allowed[rng.integers(0, allowed.size, size=size)].reshape(shape)


def bf16_bits(rng, shape, exp_lo=-3, exp_hi=1):
    """bf16 bit patterns 2^e * (1 + m/128), e uniform in [exp_lo, exp_hi], m uniform in
    [0, 127], sign uniform."""
    s = rng.integers(0, 2, size=shape, dtype=np.uint16)
    e = rng.integers(127 + exp_lo, 127 + exp_hi + 1, size=shape).astype(np.uint16)
    m = rng.integers(0, 128, size=shape, dtype=np.uint16)
    return (s << 15) | (e << 7) | m


def make_qsa(name, *, ctx, rows_per_req=1, Hq, Hkv, D=128, page=64, topk=2048, seed,
             k_exp=(4, 7), q_exp=(-3, 1), gate_exp=(-3, 2), softmax_scale=None,
             output_scale=1.0, extra_pages=0, drop_frac=0.0) -> QsaCase:
    """Requests with contexts `ctx` on pages of a shuffled pool; each request's rows select
    min(topk, ctx) distinct tokens in increasing order (the indexer's top-k output
    order), -1 padded, count in the last column.  drop_frac of the selected entries
    before the count are replaced by -1 (masked entries)."""
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in ctx]
    R = len(ctx)
    npg = [-(-c // page) for c in ctx]
    P = sum(npg) + extra_pages
    W = max(npg) if npg else 1
    kv = e4m3_codes(rng, (P, Hkv, page, 2 * D), *k_exp)
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((R, W), -1, np.int32)
    at = 0
    for b in range(R):
        table[b, :npg[b]] = perm[at:at + npg[b]]
        at += npg[b]
    rows = R * rows_per_req
    t2r = np.repeat(np.arange(R, dtype=np.int32), rows_per_req)
    ind = np.full((rows, topk + 1), -1, np.int32)
    for r in range(rows):
        c = ctx[t2r[r]]
        n = min(topk, c)
        sel = np.sort(rng.choice(c, size=n, replace=False)).astype(np.int32)
        if drop_frac > 0 and n:
            sel[rng.random(n) < drop_frac] = -1
        ind[r, :n] = sel
        ind[r, topk] = n
    q = bf16_bits(rng, (rows, Hq, D), *q_exp)
    gate = bf16_bits(rng, (rows, Hq, D), *gate_exp)
    scale = float(D) ** -0.5 if softmax_scale is None else float(softmax_scale)
    return QsaCase(name, kv, table, t2r, ind, q, gate, page, scale, float(output_scale),
                   {"seed": seed, "ctx": ctx})


def qsa_selection(case: QsaCase, seed: int) -> np.ndarray:
    """Another selection for the same requests and cache: per row, min(topk, ctx)
    distinct tokens in increasing order, count in the last column."""
    rng = np.random.default_rng(seed)
    ctx = case.meta["ctx"]
    ind = np.full_like(case.indices, -1)
    for r in range(case.rows):
        c = ctx[int(case.token_to_req[r])]
        n = min(case.topk, c)
        ind[r, :n] = np.sort(rng.choice(c, size=n, replace=False))
        ind[r, case.topk] = n
    return ind


def qsa_decode_case(seed=1050, requests=128):
    """Large-batch sparse decode: 128 requests x 1 row, contexts U[8192, 32768], Hq=32,
    Hkv=4, D=128, 64-token pages, top-2048 selected tokens per row, softmax scale
    1/sqrt(128)."""
    rng = np.random.default_rng(seed + 5)
    ctx = rng.integers(8192, 32768 + 1, size=requests)
    return make_qsa("qsa_fp8_decode_b128", ctx=ctx, Hq=32, Hkv=4, D=128, page=64, topk=2048,
                    seed=seed)
