// logits.hip -- weighted-ReLU indexer logits over a paged FP4 key cache, gfx950.
//
//   logits[t][s] = sum_h w[t][h] * max(q[t][h] . k[s], 0), -inf where s is invisible
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", TL;DR and "Fix
// (production target)": FP4 operands on the matrix cores, ReLU and head weights in the
// epilogue; "[DSv4.1] Speed up the FP4 indexer scorer...", Motivation and Accuracy
// Tests: paged keys, -inf at invisible positions.)
//
// Work split.  Query rows are grouped in row blocks of RG consecutive rows (RG = 4, 2
// or 1); the columns [0, out_cols) are cut into chunks of `ppw` key pages.  One wave
// owns one (row block, column chunk) pair and writes every logit of it, so the grid
// covers the whole [T, out_cols] output exactly once.
//
// MFMA mapping.  The contraction is [rows*heads x 128] x [128 x 16 keys].  A-tile j
// holds 16 (row, head) pairs arranged so that output lane group g = l/16 always sees
// the same query row: tile row m = 4*g' + i stands for row t0 + g' % RG and head
// (16/RG)*jj + 4*(g'/RG) + i of key head hk (j = hk * tiles_per_kv + jj).  After the
// epilogue each lane therefore holds partial head sums of one (row, key) pair; with
// RG < 4 the 4/RG lane groups of a row are added with two cross-lane steps.
//
// Keys go straight from HBM into the B operand: lane l loads the 16 bytes
// [16*(l/16), +16) of key l%16 of the tile (a wave reads 1 KB contiguous per 16-key
// tile, fully coalesced) and the one E8M0 byte that covers them.  Each key byte is
// used by exactly one wave, so no LDS staging is needed on this path.
//
// Rounding.  MXFP4: one scaled MFMA per (tile, key head) covers all 128 products.
// NVFP4: E2M1 x E4M3 is not an MX operand, so both sides are decoded exactly to fp16
// (value = E2M1 * 2^a * b, at most 6 significant bits) and four fp16 MFMAs accumulate
// in fp32.  Head sums use eight accumulators per lane (chains of at most H*RG/128
// fused multiply-adds) and a tree, which bounds the head-sum rounding well inside
// 1e-6 * sum_h |w_h ReLU(dot_h)|.  ReLU is fmaxf (IEEE maxNum: a NaN dot counts as 0).
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kWavesPerBlock = 4;

// Cross-lane sum of the 4/RG lane groups that share a row.
template <int RG>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (RG == 1) {
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
    } else if constexpr (RG == 2) {
        v += __shfl_xor(v, 32);
    }
    return v;
}

// Store one 16-key tile of results: lane (g, n) owns column s0 + n of row t (lanes of
// groups g >= RG only hold copies when RG < 4 and do not store).
template <int RG>
__device__ __forceinline__ void store_tile(const LogitsParams& p, int g, int n, int t, bool row_ok,
                                           int len, int s0, float v) {
    int s = s0 + n;
    if (g < RG && row_ok && s < p.out_cols)
        p.out[(int64_t)t * p.out_rs + s] = (s < len) ? v : -__builtin_inff();
}

// A-operand row of lane l: which (query row, head) of tile j it supplies.
template <int RG>
__device__ __forceinline__ void a_row_of_lane(const LogitsParams& p, int lane, int j, int& trow_off,
                                              int& head, bool& valid) {
    int m = lane & 15;
    int gp = m >> 2, i = m & 3;
    int hk = j / p.tiles_per_kv, jj = j - hk * p.tiles_per_kv;
    int hl = (16 / RG) * jj + 4 * (gp / RG) + i;
    trow_off = gp % RG;
    head = hk * p.R + hl;
    valid = hl < p.R;
}

// Head (within all H) whose result lands in element i of output lane group g, tile j.
template <int RG>
__device__ __forceinline__ int out_head(const LogitsParams& p, int g, int j, int i, bool& valid) {
    int hk = j / p.tiles_per_kv, jj = j - hk * p.tiles_per_kv;
    int hl = (16 / RG) * jj + 4 * (g / RG) + i;
    valid = hl < p.R;
    return hk * p.R + hl;
}

// ------------------------------------------------------------------ MXFP4 kernel
template <int RG, int NT>
__global__ __launch_bounds__(256) void k_logits_mx(const LogitsParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int rb = gw / p.n_wchunks;
    const int wc = gw - rb * p.n_wchunks;
    if (rb >= p.n_rowblocks) return;  // uniform per wave
    const int g = lane >> 4, n = lane & 15;
    const int t0 = rb * RG;
    const int t_last = min(t0 + RG, p.T) - 1;
    const int n_pages_out = (p.out_cols + p.page - 1) / p.page;
    const int lp_begin = wc * p.ppw;
    const int lp_end = min(lp_begin + p.ppw, n_pages_out);

    // The rows of a block may belong to different requests; each pass handles the rows
    // of one request (rows of a request are consecutive).
    int t_seg = t0;
    while (t_seg <= t_last) {
        const int b = uniform(find_request(p.cu, p.B, t_seg));
        // rows past cu_seqlens_q[B] belong to no request: they see nothing
        const bool req_ok = t_seg < p.cu[b + 1];
        const int seg_end = req_ok ? uniform(min(p.cu[b + 1], t_last + 1)) : t_last + 1;
        const int t_next = seg_end;

        // ---- query operands, weights and lengths of this segment
        v4i a[NT];
        int sa[NT];
        float wv[NT][4];
#pragma unroll
        for (int j = 0; j < NT; j++) {
            int toff, head;
            bool ok;
            a_row_of_lane<RG>(p, lane, j, toff, head, ok);
            int t = t0 + toff;
            ok = ok && j < p.n_tiles && req_ok && t >= t_seg && t < seg_end;
            if (ok) {
                a[j] = load16(p.q + (int64_t)t * p.q_rs + (int64_t)head * 64 + 16 * (lane >> 4));
                sa[j] = p.qs[(int64_t)t * p.qs_rs + (int64_t)head * 4 + (lane >> 4)];
            } else {
                a[j] = v4i{0, 0, 0, 0};
                sa[j] = 127;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bool hv;
                int h = out_head<RG>(p, g, j, i, hv);
                int to = t0 + (g % RG);
                hv = hv && j < p.n_tiles && req_ok && to >= t_seg && to < seg_end;
                wv[j][i] = hv ? p.w[(int64_t)to * p.w_rs + h] : 0.0f;
            }
        }
        const int t_out = t0 + (g % RG);
        const bool row_ok = t_out >= t_seg && t_out < seg_end;
        int len = (row_ok && req_ok) ? min(p.lens[t_out], p.out_cols) : 0;
        // longest visible length among the segment's rows (wave-uniform)
        int max_len = len;
        max_len = max(max_len, __shfl_xor(max_len, 16));
        max_len = max(max_len, __shfl_xor(max_len, 32));
        max_len = uniform(max_len);

        for (int lp = lp_begin; lp < lp_end; lp++) {
            const int col0 = lp * p.page;
            int phys = -1;
            if (req_ok && col0 < max_len && lp < p.W) phys = uniform(p.bt[(int64_t)b * p.bt_rs + lp]);
            const bool page_ok = phys >= 0 && phys < p.num_pages;
            for (int tt = 0; tt < p.page / 16; tt++) {
                const int s0 = col0 + tt * 16;
                if (!page_ok) {
                    store_tile<RG>(p, g, n, t_out, row_ok, 0, s0, 0.0f);
                    continue;
                }
                float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                for (int hk = 0; hk < p.Hkv; hk++) {
                    const int64_t tok = (int64_t)hk * p.page + tt * 16 + n;
                    const v4i kb = load16(p.k + (int64_t)phys * p.kp_s + tok * 64 + 16 * (lane >> 4));
                    const int sk = p.ks[(int64_t)phys * p.ksp_s + tok * 4 + (lane >> 4)];
#pragma unroll
                    for (int j = 0; j < NT; j++) {
                        if (j >= p.n_tiles || j / p.tiles_per_kv != hk) continue;
                        v4f d = mfma_fp4_16x16x128(a[j], sa[j], kb, sk, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[j & 1][i] = __builtin_fmaf(wv[j][i], fmaxf(d[i], 0.0f), acc[j & 1][i]);
                    }
                }
                float v = ((acc[0][0] + acc[0][1]) + (acc[0][2] + acc[0][3])) +
                          ((acc[1][0] + acc[1][1]) + (acc[1][2] + acc[1][3]));
                v = group_sum<RG>(v);
                store_tile<RG>(p, g, n, t_out, row_ok, len, s0, v);
            }
        }
        t_seg = t_next;
    }
}

// ------------------------------------------------------------------ NVFP4 kernel
// Same work split; operands are decoded exactly to fp16 (see the file comment).  Lane
// l's 16 bytes [16*(l/16), +16) hold elements [32*(l/16), +32); dword c of them feeds
// MFMA chunk c, and those 8 elements lie in scale group 2*(l/16) + c/2.
template <int RG, int NT>
__global__ __launch_bounds__(256) void k_logits_nv(const LogitsParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int rb = gw / p.n_wchunks;
    const int wc = gw - rb * p.n_wchunks;
    if (rb >= p.n_rowblocks) return;
    const int g = lane >> 4, n = lane & 15;
    const int t0 = rb * RG;
    const int t_last = min(t0 + RG, p.T) - 1;
    const int n_pages_out = (p.out_cols + p.page - 1) / p.page;
    const int lp_begin = wc * p.ppw;
    const int lp_end = min(lp_begin + p.ppw, n_pages_out);

    int t_seg = t0;
    while (t_seg <= t_last) {
        const int b = uniform(find_request(p.cu, p.B, t_seg));
        // rows past cu_seqlens_q[B] belong to no request: they see nothing
        const bool req_ok = t_seg < p.cu[b + 1];
        const int seg_end = req_ok ? uniform(min(p.cu[b + 1], t_last + 1)) : t_last + 1;
        const int t_next = seg_end;

        v8h a[NT][4];
        float wv[NT][4];
#pragma unroll
        for (int j = 0; j < NT; j++) {
            int toff, head;
            bool ok;
            a_row_of_lane<RG>(p, lane, j, toff, head, ok);
            int t = t0 + toff;
            ok = ok && j < p.n_tiles && req_ok && t >= t_seg && t < seg_end;
            v4i raw = v4i{0, 0, 0, 0};
            uint32_t sc = 0;
            if (ok) {
                raw = load16(p.q + (int64_t)t * p.q_rs + (int64_t)head * 64 + 16 * (lane >> 4));
                const uint8_t* sp = p.qs + (int64_t)t * p.qs_rs + (int64_t)head * 8 + 2 * (lane >> 4);
                sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
            }
#pragma unroll
            for (int c = 0; c < 4; c++) {
                float pw, bb;
                e4m3_split((sc >> (8 * (c >> 1))) & 0xffu, pw, bb);
                a[j][c] = decode8_f16((uint32_t)raw[c], pw, bb);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bool hv;
                int h = out_head<RG>(p, g, j, i, hv);
                int to = t0 + (g % RG);
                hv = hv && j < p.n_tiles && req_ok && to >= t_seg && to < seg_end;
                wv[j][i] = hv ? p.w[(int64_t)to * p.w_rs + h] : 0.0f;
            }
        }
        const int t_out = t0 + (g % RG);
        const bool row_ok = t_out >= t_seg && t_out < seg_end;
        int len = (row_ok && req_ok) ? min(p.lens[t_out], p.out_cols) : 0;
        int max_len = len;
        max_len = max(max_len, __shfl_xor(max_len, 16));
        max_len = max(max_len, __shfl_xor(max_len, 32));
        max_len = uniform(max_len);

        for (int lp = lp_begin; lp < lp_end; lp++) {
            const int col0 = lp * p.page;
            int phys = -1;
            if (req_ok && col0 < max_len && lp < p.W) phys = uniform(p.bt[(int64_t)b * p.bt_rs + lp]);
            const bool page_ok = phys >= 0 && phys < p.num_pages;
            for (int tt = 0; tt < p.page / 16; tt++) {
                const int s0 = col0 + tt * 16;
                if (!page_ok) {
                    store_tile<RG>(p, g, n, t_out, row_ok, 0, s0, 0.0f);
                    continue;
                }
                float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                for (int hk = 0; hk < p.Hkv; hk++) {
                    const int64_t tok = (int64_t)hk * p.page + tt * 16 + n;
                    const v4i kr = load16(p.k + (int64_t)phys * p.kp_s + tok * 64 + 16 * (lane >> 4));
                    const uint8_t* sp = p.ks + (int64_t)phys * p.ksp_s + tok * 8 + 2 * (lane >> 4);
                    const uint32_t sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
                    v8h kb[4];
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        float pw, bb;
                        e4m3_split((sc >> (8 * (c >> 1))) & 0xffu, pw, bb);
                        kb[c] = decode8_f16((uint32_t)kr[c], pw, bb);
                    }
#pragma unroll
                    for (int j = 0; j < NT; j++) {
                        if (j >= p.n_tiles || j / p.tiles_per_kv != hk) continue;
                        v4f d = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < 4; c++) d = mfma_f16_16x16x32(a[j][c], kb[c], d);
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[j & 1][i] = __builtin_fmaf(wv[j][i], fmaxf(d[i], 0.0f), acc[j & 1][i]);
                    }
                }
                float v = ((acc[0][0] + acc[0][1]) + (acc[0][2] + acc[0][3])) +
                          ((acc[1][0] + acc[1][1]) + (acc[1][2] + acc[1][3]));
                v = group_sum<RG>(v);
                store_tile<RG>(p, g, n, t_out, row_ok, len, s0, v);
            }
        }
        t_seg = t_next;
    }
}

template <int RG, int NT>
hipError_t launch_rg_nt(const LogitsParams& p, hipStream_t stream) {
    int64_t waves = (int64_t)p.n_rowblocks * p.n_wchunks;
    int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks <= 0) return hipSuccess;
    if (p.fmt == 0)
        hipLaunchKernelGGL((k_logits_mx<RG, NT>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((k_logits_nv<RG, NT>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int RG>
hipError_t launch_rg(const LogitsParams& p, hipStream_t stream) {
    if (p.n_tiles <= 2) return launch_rg_nt<RG, 2>(p, stream);
    if (p.n_tiles <= 4) return launch_rg_nt<RG, 4>(p, stream);
    if (p.n_tiles <= 8) return launch_rg_nt<RG, 8>(p, stream);
    return launch_rg_nt<RG, 16>(p, stream);
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p_in, hipStream_t stream) {
    LogitsParams p = p_in;
    // Rows per A-tile group: as many as the average request holds (up to 4), reduced
    // while the A tiles would not fit the register budget.  Any choice is correct; rows
    // of different requests in one block are handled in separate passes.
    int rg = 1;
    if (p.T >= 4 * p.B) rg = 4;
    else if (p.T >= 2 * p.B) rg = 2;
    const int nt_cap = p.fmt == 0 ? 16 : 8;
    for (;;) {
        int hpt = 16 / rg;  // heads per A tile per row
        p.tiles_per_kv = (p.R + hpt - 1) / hpt;
        p.n_tiles = p.Hkv * p.tiles_per_kv;
        if (p.n_tiles <= nt_cap || rg == 1) break;
        rg >>= 1;
    }
    if (p.n_tiles > 16) return hipErrorInvalidValue;  // guarded by the host checks
    p.rows_per_block = rg;
    p.n_rowblocks = (p.T + rg - 1) / rg;
    const int n_pages_out = (p.out_cols + p.page - 1) / p.page;
    // pages per wave: enough waves to cover the chip a few times over
    int64_t total = (int64_t)p.n_rowblocks * n_pages_out;
    int64_t ppw = (total + 8191) / 8192;
    if (ppw < 1) ppw = 1;
    if (ppw > 64) ppw = 64;
    p.ppw = (int)ppw;
    p.n_wchunks = (n_pages_out + p.ppw - 1) / p.ppw;
    if (p.n_wchunks == 0 || p.n_rowblocks == 0) return hipSuccess;
    switch (rg) {
        case 4: return launch_rg<4>(p, stream);
        case 2: return launch_rg<2>(p, stream);
        default: return launch_rg<1>(p, stream);
    }
}

}  // namespace fp4idx
