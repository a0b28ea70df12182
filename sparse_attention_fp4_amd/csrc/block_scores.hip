// block_scores.hip -- per-head 128-token block-max QK scores over paged FP4 keys, gfx950.
//
//   scores[hq][kb][q] = max over valid keys k in [128 kb, 128 kb + 128) of q . k
//
// ("M3 FP4 Indexer" README, 数学语义 and the causal paragraph after it: bottom-right
// causal offset k_len - q_len unless qo_offset is given; keys past k_len never count;
// an empty block is -inf.)
//
// Work split: one wave owns 16 consecutive query tokens (a query tile), up to NB query
// heads of one key-head group and a chunk of kb_chunk consecutive 128-key blocks; it
// walks the key tiles of its chunk that the tile can see in 16-key steps and writes
// every score block of its chunk for its (heads, tokens), including the -inf blocks it
// never reaches.  Cutting the key range keeps the waves' work even under the causal
// mask (late query tiles see many more keys) and the grid many times the chip's size.
// Query tiles that straddle two batch items are handled one item at a time.
//
// MFMA mapping: A = 16 keys x 128, B = 128 x 16 query tokens of one head, so output
// lane (g, n) holds keys 4g..4g+3 of the tile for token n.  The block max is a running
// max over tiles in each lane, then two cross-lane steps (over the four lane groups)
// at each 128-key block boundary; lane group 0 stores 16 consecutive tokens (64 B).
//
// Key tiles are fetched two ahead of the one being computed, through buffer
// descriptors built per tile (an invalid page gets a zero-byte descriptor, so the
// loads stay unconditional); the block-table entries of 64 blocks come in with one
// load.  NVFP4 workgroups whose 64 tokens lie in one batch item instead walk whole
// 128-key blocks in step and decode each block once into LDS for their four waves
// (block_scores_shared below).
//
// MXFP4 uses the scaled FP4 MFMA (one instruction per 16x16 tile covers all 128
// products).  NVFP4 decodes both operands exactly to fp16 (E2M1 * 2^a * b, b the E4M3
// significand as an integer) and accumulates four 16x16x32 fp16 MFMAs in fp32.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kXcdRun = 32;     // consecutive workgroups kept on one XCD
constexpr int kChunkNv = 8;     // 128-key blocks per NVFP4 wave
constexpr int kChunkMx = 16;    // 128-key blocks per MXFP4 wave

template <int FMT>
struct QOperand;

template <>
struct QOperand<0> {
    v4i v;
    int s;
};

template <>
struct QOperand<1> {
    v8h v[4];
};

// max of three floats; fmax skips a NaN operand (the block max's reading of fmax)
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// NVFP4, the four query tiles of a workgroup in one batch item: the waves walk the same
// 128-key blocks in step and share their decoding.  Per block, wave w loads and decodes
// key tiles w and w + 4 (16 keys each) to fp16 in LDS; after a barrier every wave reads
// all eight tiles as MFMA operands for its own query tile.  A quarter of the decoding and
// of the key reads per wave, one buffer descriptor and one block-table lookup per block;
// the next block's bytes are loaded while the current one is computed.  With one LDS
// buffer (32 KB: three workgroups per CU) a second barrier per block guards its reuse;
// two buffers need one barrier but leave room for two workgroups, which measured slower.
// A wave whose own keys end earlier keeps decoding for the others.
template <int NB>
__device__ __forceinline__ void block_scores_shared(const BlockParams& p, int hk, int kc, int h0,
                                                    int nh, int qt, int b, int t_last,
                                                    v8h (*sk)[4][64]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int kb_lo = kc * p.kb_chunk;
    const int kb_hi = min(kb_lo + p.kb_chunk, p.ktiles);
    const int cq0 = p.cu_q[b], cq1 = p.cu_q[b + 1];
    const int q_len = cq1 - cq0;
    const int k_len = min(p.cu_k[b + 1] - p.cu_k[b], p.ktiles * 128);
    const int offset = p.qo_offset ? p.qo_offset[b] : (p.cu_k[b + 1] - p.cu_k[b]) - q_len;
    const int page0 = p.cu_p[b];
    const int qg = qt * 16 + n;
    const bool col_ok = qg <= t_last;  // the workgroup's tokens up to t_last are all in batch item b
    auto visible = [&](int t) {        // keys visible to token t of batch item b (exclusive bound)
        return p.causal ? min(k_len, max(t - cq0 + offset + 1, 0)) : k_len;
    };
    const int kv_lim = col_ok ? visible(qg) : 0;
    int kv_max = kv_lim;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) kv_max = max(kv_max, __shfl_xor(kv_max, d));
    kv_max = uniform(kv_max);
    int kv_min = col_ok ? kv_lim : 0x7fffffff;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) kv_min = min(kv_min, __shfl_xor(kv_min, d));
    kv_min = uniform(kv_min);

    QOperand<1> qop[NB];
#pragma unroll
    for (int hb = 0; hb < NB; hb++) {
        const bool ok = col_ok && hb < nh;
        const int64_t row = (int64_t)qg * p.Hq + h0 + hb;
        v4i raw = v4i{0, 0, 0, 0};
        uint32_t sc = 0;
        if (ok) {
            raw = load16(p.q + row * 64 + 16 * g);
            sc = (uint32_t)p.qs[row * 8 + 2 * g] | ((uint32_t)p.qs[row * 8 + 2 * g + 1] << 8);
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            float pw, bb;
            e4m3_split((sc >> (8 * (c >> 1))) & 0xffu, pw, bb);
            qop[hb].v[c] = decode8_f16((uint32_t)raw[c], pw, bb);
        }
    }

    const int n_kt = (kv_max + 15) / 16;        // this wave's key tiles with a visible key
    const int kb_done = (n_kt + 7) / 8;         // and its blocks
    // the workgroup walks the blocks of its last token (visibility grows with the token)
    const int kb_done_wg = (visible(t_last) + 127) / 128;
    const int wkb_hi = min(kb_hi, kb_done_wg);
    float run[NB];

    int win = -64 - 64, my_phys = -1;
    auto window = [&](int kb) {
        if (kb - win >= 64 || kb < win) {
            win = kb & ~63;
            const int i = win + lane;
            int v = -1;
            if (p.kv_indices && i < kb_done_wg) v = p.kv_indices[page0 + i];
            my_phys = (v >= 0 && v < p.num_pages) ? v : -1;
        }
        return __builtin_amdgcn_readlane(my_phys, kb - win);
    };
    // this wave's two tiles of block kb (w and w + 4): lane (g, n) holds the 16 bytes of
    // key n, dims 32g..32g+31, and their two scale codes
    struct KBlk {
        v4i k0, k1;
        uint32_t s0, s1;
        int phys;
    };
    auto fetch = [&](int kb, KBlk& t) {
        t.phys = kb < wkb_hi ? window(kb) : -1;
        const bool ok = t.phys >= 0;
        const int64_t tok0 = ((int64_t)(ok ? t.phys : 0) * p.Hkv + hk) * 128;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(ok ? p.k + tok0 * 64 : p.k, ok ? 128u * 64u : 0u);
        const int koff = (wave * 16 + n) * 64 + 16 * g;
        t.k0 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 0, 0));
        t.k1 = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 4 * 16 * 64, 0));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(ok ? p.ks + tok0 * 8 : p.ks, ok ? 128u * 8u : 0u);
        const int soff = (wave * 16 + n) * 8 + 2 * g;
        t.s0 = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
        t.s1 = __builtin_amdgcn_raw_buffer_load_b16(rs, soff + 4 * 16 * 8, 0, 0);
    };
    auto stage = [&](const v4i& k, uint32_t sc, v8h (*tile)[64]) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            float pw, bb;
            e4m3_split((sc >> (8 * (c >> 1))) & 0xffu, pw, bb);
            tile[c][lane] = decode8_f16((uint32_t)k[c], pw, bb);  // zeros for an invalid page
        }
    };
    auto block = [&](int kb, const KBlk& t) {
        // one 32 KB tile (three workgroups per CU; two buffers measured slower): wait
        // until every wave is done with the previous block
        v8h (*buf)[4][64] = sk;
        __syncthreads();
        stage(t.k0, t.s0, buf[wave]);
        stage(t.k1, t.s1, buf[wave + 4]);
        __syncthreads();
        if (kb < kb_lo || kb >= kb_done) return;  // wave-uniform: no key of this block is visible
#pragma unroll
        for (int hb = 0; hb < NB; hb++) run[hb] = -__builtin_inff();
        if (t.phys >= 0) {
            const int nt = min(8, n_kt - kb * 8);            // tiles with a visible key
            const bool full = kb * 128 + 128 <= kv_min;      // every key of the block visible
#pragma unroll
            for (int j = 0; j < 8; j++) {
                if (j >= nt) break;
                v8h kd[4];
#pragma unroll
                for (int c = 0; c < 4; c++) kd[c] = buf[j][c][lane];
                v4f d[NB];
#pragma unroll
                for (int hb = 0; hb < NB; hb++) d[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; c++)
#pragma unroll
                    for (int hb = 0; hb < NB; hb++) d[hb] = mfma_f16_16x16x32(kd[c], qop[hb].v[c], d[hb]);
                if (__builtin_expect(full, 1)) {
#pragma unroll
                    for (int hb = 0; hb < NB; hb++)
                        run[hb] = max3_raw(max3_raw(run[hb], d[hb][0], d[hb][1]), d[hb][2], d[hb][3]);
                } else {
                    const int kbase = kb * 128 + j * 16 + 4 * g;
#pragma unroll
                    for (int hb = 0; hb < NB; hb++) {
                        v4f e = d[hb];
#pragma unroll
                        for (int i = 0; i < 4; i++) e[i] = kbase + i < kv_lim ? e[i] : -__builtin_inff();
                        run[hb] = max3_raw(max3_raw(run[hb], e[0], e[1]), e[2], e[3]);
                    }
                }
            }
        }
#pragma unroll
        for (int hb = 0; hb < NB; hb++) {
            float v = run[hb];
            v = max_lane_xor16(v);
            v = max_lane_xor32(v);
            if (g == 0 && col_ok && hb < nh) p.scores[((int64_t)(h0 + hb) * p.ktiles + kb) * p.Tq + qg] = v;
        }
    };
    // the loop bound is the workgroup's: every wave takes every barrier
    KBlk A, B;
    fetch(kb_lo, A);
    for (int kb = kb_lo; kb < wkb_hi; kb += 2) {
        fetch(kb + 1, B);
        block(kb, A);
        if (kb + 1 >= wkb_hi) break;
        fetch(kb + 2, A);
        block(kb + 1, B);
    }
    // blocks of the chunk this wave never reached: -inf
    for (int kb = max(kb_done, kb_lo); kb < kb_hi; kb++) {
        if (g == 0 && col_ok) {
#pragma unroll
            for (int hb = 0; hb < NB; hb++)
                if (hb < nh) p.scores[((int64_t)(h0 + hb) * p.ktiles + kb) * p.Tq + qg] = -__builtin_inff();
        }
    }
}

template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_block_scores(const BlockParams p) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int n_qtiles = (p.Tq + 15) / 16;
    const int n_hgrp = (p.R + NB - 1) / NB;
    // block index -> (kv head, key chunk, head group, 4 consecutive query tiles); the
    // query tiles of one key chunk are neighbours, so their key reads meet in L2 -- and
    // runs of 32 neighbours go to one XCD, whose L2 is its own (half the HBM fetches of
    // dispatch order, same time)
    const int qt_blocks = (n_qtiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int per_hk = p.n_kchunks * n_hgrp * qt_blocks;
    const int bx = xcd_order(blockIdx.x, kXcdRun);
    if (bx >= p.Hkv * per_hk) return;  // grid padding
    const int hk = bx / per_hk;
    int rem = bx - hk * per_hk;
    const int kc = rem / (n_hgrp * qt_blocks);
    rem -= kc * n_hgrp * qt_blocks;
    const int hgrp = rem / qt_blocks;
    const int qt = (rem - hgrp * qt_blocks) * kWavesPerBlock + (threadIdx.x >> 6);
    if constexpr (FMT == 1) {
        // the workgroup's 64 tokens in one batch item: shared key decoding
        __shared__ __align__(16) v8h sk[8][4][64];
        const int qt0 = (rem - hgrp * qt_blocks) * kWavesPerBlock;
        const int t_first = qt0 * 16, t_last = min(qt0 * 16 + 64, p.Tq) - 1;
        const RowRequest ra = find_request(p.cu_q, p.B, t_first);
        const RowRequest rb = find_request(p.cu_q, p.B, t_last);
        if (hk < p.Hkv && ra.ok && rb.ok && ra.b == rb.b) {  // uniform per workgroup
            block_scores_shared<NB>(p, hk, kc, hk * p.R + hgrp * NB, min(NB, p.R - hgrp * NB), qt,
                                    ra.b, t_last, sk);
            return;
        }
    }
    if (hk >= p.Hkv || qt >= n_qtiles) return;  // uniform per wave
    const int kb_lo = kc * p.kb_chunk;                       // this wave's blocks
    const int kb_hi = min(kb_lo + p.kb_chunk, p.ktiles);
    const int h0 = hk * p.R + hgrp * NB;         // first query head of this wave
    const int nh = min(NB, p.R - hgrp * NB);
    const int q_first = qt * 16;
    const int q_lastp1 = min(q_first + 16, p.Tq);

    int q_seg = q_first;
    while (q_seg < q_lastp1) {
        const RowRequest rq = find_request(p.cu_q, p.B, q_seg);
        const int b = rq.b;
        const int cq0 = p.cu_q[b], cq1 = p.cu_q[b + 1];
        const bool req_ok = rq.ok;
        const int seg_end = req_ok ? min(cq1, q_lastp1) : q_lastp1;
        const int q_len = cq1 - cq0;
        // keys past the output's Ktiles*128 columns have no block to land in
        const int k_len = req_ok ? min(p.cu_k[b + 1] - p.cu_k[b], p.ktiles * 128) : 0;
        const int offset = p.qo_offset ? p.qo_offset[b] : (p.cu_k[b + 1] - p.cu_k[b]) - q_len;
        const int page0 = p.cu_p[b];
        // token of this lane's B column and its visible key bound (exclusive)
        const int qg = q_first + n;
        const bool col_ok = qg >= q_seg && qg < seg_end;
        const int q_local = qg - cq0;
        int kv_lim = k_len;
        if (p.causal) kv_lim = min(kv_lim, max(q_local + offset + 1, 0));
        if (!col_ok) kv_lim = 0;
        // wave-wide bound: largest kv_lim over the columns
        int kv_max = kv_lim;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) kv_max = max(kv_max, __shfl_xor(kv_max, d));
        kv_max = uniform(kv_max);
        int kv_min = col_ok ? kv_lim : 0x7fffffff;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) kv_min = min(kv_min, __shfl_xor(kv_min, d));
        kv_min = uniform(kv_min);

        // query operands (B): token qg, head h0 + hb
        QOperand<FMT> qop[NB];
#pragma unroll
        for (int hb = 0; hb < NB; hb++) {
            const bool ok = col_ok && hb < nh;
            const int hq = h0 + hb;
            const int64_t row = (int64_t)qg * p.Hq + hq;
            if constexpr (FMT == 0) {
                if (ok) {
                    qop[hb].v = load16(p.q + row * 64 + 16 * g);
                    qop[hb].s = p.qs[row * 4 + g];
                } else {
                    qop[hb].v = v4i{0, 0, 0, 0};
                    qop[hb].s = 127;
                }
            } else {
                v4i raw = v4i{0, 0, 0, 0};
                uint32_t sc = 0;
                if (ok) {
                    raw = load16(p.q + row * 64 + 16 * g);
                    sc = (uint32_t)p.qs[row * 8 + 2 * g] | ((uint32_t)p.qs[row * 8 + 2 * g + 1] << 8);
                }
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    float pw, bb;
                    e4m3_split((sc >> (8 * (c >> 1))) & 0xffu, pw, bb);
                    qop[hb].v[c] = decode8_f16((uint32_t)raw[c], pw, bb);
                }
            }
        }

        const int n_kt = (kv_max + 15) / 16;      // key tiles with any visible key
        const int kb_done = (n_kt + 7) / 8;        // blocks with a visible key
        const int kt_lo = min(kb_lo * 8, n_kt);    // this wave's key tiles
        const int kt_hi = min(kb_hi * 8, n_kt);
        float run[NB];
#pragma unroll
        for (int hb = 0; hb < NB; hb++) run[hb] = -__builtin_inff();

        // Block-table entries of 64 blocks at a time: lane i holds the page of block
        // win + i (-1 when invalid).  Key tiles are fetched two ahead of the one being
        // computed, through buffer descriptors that read zeros for invalid pages.
        int win = -64 - 64, my_phys = -1;
        auto window = [&](int kb) {
            if (kb - win >= 64 || kb < win) {
                win = kb & ~63;
                const int i = win + lane;
                int v = -1;
                if (p.kv_indices && i < kb_done) v = p.kv_indices[page0 + i];
                my_phys = (v >= 0 && v < p.num_pages) ? v : -1;
            }
            return __builtin_amdgcn_readlane(my_phys, kb - win);
        };
        struct KTile {
            v4i k;
            uint32_t s;
            int phys;
        };
        auto fetch = [&](int kt, KTile& t) {
            t.phys = kt < kt_hi ? window(kt >> 3) : -1;
            const bool ok = t.phys >= 0;
            const int64_t tok0 = ((int64_t)(ok ? t.phys : 0) * p.Hkv + hk) * 128 + (kt & 7) * 16;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(ok ? p.k + tok0 * 64 : p.k, ok ? 16u * 64u : 0u);
            t.k = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, n * 64 + 16 * g, 0, 0));
            constexpr int G = FMT == 0 ? 4 : 8;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(ok ? p.ks + tok0 * G : p.ks, ok ? 16u * G : 0u);
            if constexpr (FMT == 0)
                t.s = __builtin_amdgcn_raw_buffer_load_b8(rs, n * 4 + g, 0, 0);
            else
                t.s = __builtin_amdgcn_raw_buffer_load_b16(rs, n * 8 + 2 * g, 0, 0);
        };
        auto process = [&](int kt, const KTile& t) {
            const int kb = kt >> 3;
            if (t.phys >= 0) {
                // keys of this lane's output rows: kt*16 + 4g + i.  Heads past nh have
                // zero query operands and are computed but never stored, so the head
                // loop has no branch; the products of all heads are independent.
                const int kbase = kt * 16 + 4 * g;
                const bool full = __ballot(kbase + 3 >= kv_min) == 0;  // whole tile visible
                v4f d[NB];
                if constexpr (FMT == 0) {
#pragma unroll
                    for (int hb = 0; hb < NB; hb++)
                        d[hb] = mfma_fp4_16x16x128(t.k, (int)t.s, qop[hb].v, qop[hb].s, v4f{0.f, 0.f, 0.f, 0.f});
                } else {
                    v8h kd[4];
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        float pw, bb;
                        e4m3_split((t.s >> (8 * (c >> 1))) & 0xffu, pw, bb);
                        kd[c] = decode8_f16((uint32_t)t.k[c], pw, bb);
                    }
#pragma unroll
                    for (int hb = 0; hb < NB; hb++) d[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 4; c++)
#pragma unroll
                        for (int hb = 0; hb < NB; hb++) d[hb] = mfma_f16_16x16x32(kd[c], qop[hb].v[c], d[hb]);
                }
                if (__builtin_expect(full, 1)) {
#pragma unroll
                    for (int hb = 0; hb < NB; hb++)
                        run[hb] = max3_raw(max3_raw(run[hb], d[hb][0], d[hb][1]), d[hb][2], d[hb][3]);
                } else {
#pragma unroll
                    for (int hb = 0; hb < NB; hb++) {
                        v4f e = d[hb];
#pragma unroll
                        for (int i = 0; i < 4; i++) e[i] = kbase + i < kv_lim ? e[i] : -__builtin_inff();
                        run[hb] = max3_raw(max3_raw(run[hb], e[0], e[1]), e[2], e[3]);
                    }
                }
            }
            // block boundary: reduce over the four lane groups and store
            if ((kt & 7) == 7 || kt == n_kt - 1) {
#pragma unroll
                for (int hb = 0; hb < NB; hb++) {
                    float v = run[hb];
                    v = max_lane_xor16(v);
                    v = max_lane_xor32(v);
                    if (g == 0 && col_ok && hb < nh)
                        p.scores[((int64_t)(h0 + hb) * p.ktiles + kb) * p.Tq + qg] = v;
                    run[hb] = -__builtin_inff();
                }
            }
        };
        KTile t0, t1, t2;
        fetch(kt_lo, t0);
        fetch(kt_lo + 1, t1);
        for (int kt = kt_lo; kt < kt_hi; kt += 3) {
            fetch(kt + 2, t2);
            process(kt, t0);
            if (kt + 1 >= kt_hi) break;
            fetch(kt + 3, t0);
            process(kt + 1, t1);
            if (kt + 2 >= kt_hi) break;
            fetch(kt + 4, t1);
            process(kt + 2, t2);
        }
        // blocks of the chunk never reached: -inf
        for (int kb = max(kb_done, kb_lo); kb < kb_hi; kb++) {
            if (g == 0 && col_ok) {
#pragma unroll
                for (int hb = 0; hb < NB; hb++)
                    if (hb < nh) p.scores[((int64_t)(h0 + hb) * p.ktiles + kb) * p.Tq + qg] = -__builtin_inff();
            }
        }
        q_seg = seg_end;
    }
}

template <int FMT, int NB>
hipError_t launch_fmt_nb(const BlockParams& p, hipStream_t stream) {
    const int n_qtiles = (p.Tq + 15) / 16;
    const int n_hgrp = (p.R + NB - 1) / NB;
    const int qt_blocks = (n_qtiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t blocks = (int64_t)p.Hkv * p.n_kchunks * n_hgrp * qt_blocks;
    if (blocks <= 0) return hipSuccess;
    const int64_t grid = xcd_grid(blocks, kXcdRun);
    hipLaunchKernelGGL((k_block_scores<FMT, NB>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_scores(const BlockParams& p_in, hipStream_t stream) {
    BlockParams p = p_in;
    p.kb_chunk = p.fmt == 0 ? kChunkMx : kChunkNv;
    p.n_kchunks = (p.ktiles + p.kb_chunk - 1) / p.kb_chunk;
    if (p.n_kchunks == 0) p.n_kchunks = 1;  // no blocks: the grid still runs its (empty) chunk
    if (p.fmt == 0) {
        if (p.R <= 4) return launch_fmt_nb<0, 4>(p, stream);
        if (p.R <= 8) return launch_fmt_nb<0, 8>(p, stream);
        return launch_fmt_nb<0, 16>(p, stream);
    }
    // NVFP4 keeps its query operands decoded to fp16 (16 registers per head): four
    // heads per wave leave room for three waves per SIMD
    return launch_fmt_nb<1, 4>(p, stream);
}

}  // namespace fp4idx
