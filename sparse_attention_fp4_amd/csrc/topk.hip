// topk.hip -- exact top-k selection over score rows, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Order: larger score first, ties to the smaller column; -inf and NaN are never
// selected; -0 equals +0.  Output: the selected columns in increasing order, padded
// with -1.
//
// Method (rows of at most 32768 columns; longer rows, and a few rows of more than 8192,
// go to topk_long.hip): radix-style
// select on order-preserving 32-bit keys held in registers.  One workgroup (16 waves,
// 1024 lanes) takes one row: lane x holds elements x, x + 1024, x + 2048, ... loaded in
// one burst.  It narrows the key range [lo, hi] that holds the k-th largest key with
// 4096-bin LDS histograms whose bins split the current range into equal power-of-two
// widths (the first range is the observed min..max of the valid keys, so clustered
// scores still spread over many bins); the bin holding the k-th key is found by a
// block-wide scan over the bin counts.  At most three passes reach a single key T, and
// the counts give the number of ties at T to keep.  The selected elements are then
// compacted in index order: a 64-element step of one wave covers 64 consecutive
// indices, ballots give each lane its rank inside the step, and a scan over the
// (step, wave) counts gives each step its output offset.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxElems = 32768;          // columns of a row held by one workgroup
constexpr int kPer = kMaxElems / kThreads;
constexpr int kBins = 4096;
constexpr int kBinBits = 12;

// Order-preserving key: larger float -> larger key; -0 -> +0; -inf, NaN -> 0 (never
// selected: every selectable key is at least key(-FLT_MAX) = 0x00800000).
__device__ __forceinline__ uint32_t to_key(float v) {
    if (!(v > -__builtin_inff())) return 0u;
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of to_key for selectable keys.
__device__ __forceinline__ float from_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kRankMax = 1024;  // threshold-bin candidates ranked by direct comparison

struct Shared {
    alignas(16) uint32_t hist[kBins];  // read 16 bytes at a time by the bin picks
    uint32_t mkey[kRankMax];     // candidates in the threshold bin of the value pass
    int midx[kRankMax];
    int nm;
    uint32_t T;
    int need;
    uint32_t blo, bhi;
    int cnt_gt[kPer * kWaves];   // per (step j, wave w), index e = j * kWaves + w
    int cnt_eq[kPer * kWaves];
    int off_sel[kPer * kWaves];
    int off_tie[kPer * kWaves];
    uint32_t wave_min[kWaves];
    uint32_t wave_max[kWaves];
    int wave_cnt[kWaves];
    int wtot[kWaves];
    int pick[4];
    int total;
};

// Thread t's bins for a pick from the top: the kPickPer words ending at bin
// kBins - 1 - kPickPer * t, read 16 bytes at a time (one word per read would put the
// threads' bins, kPickPer words apart, in few LDS banks); c[b] / bin[b] in descending
// bin order.
constexpr int kPickPer = kBins / kThreads;
static_assert(kPickPer % 4 == 0, "whole 16-byte reads");
__device__ __forceinline__ void read_bins_desc(const uint32_t* hist, int tid, int (&c)[kPickPer],
                                               int (&bin)[kPickPer]) {
    const int lo_bin = kBins - kPickPer * (tid + 1);
    const v4u* hv = reinterpret_cast<const v4u*>(hist + lo_bin);
#pragma unroll
    for (int q = 0; q < kPickPer / 4; q++) {
        const v4u v = hv[q];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            bin[kPickPer - 1 - (4 * q + e)] = lo_bin + 4 * q + e;
            c[kPickPer - 1 - (4 * q + e)] = (int)v[e];
        }
    }
}

__device__ __forceinline__ void clear_hist(Shared& sh) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0u;
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(kThreads) void k_topk(const TopkParams p) {
    constexpr int PER = kPer;
    __shared__ Shared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    if (row >= p.rows) return;
    const int k = p.k;

    // ---- load: lane tid holds elements tid + kThreads * j
    uint32_t key[PER];
    int n = p.cols;
    if (p.row_lens) n = min(max(p.row_lens[row], 0), p.cols);
    {
        const float* src = p.scores + (int64_t)row * p.row_stride;
        float v[PER];
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const int i = tid + kThreads * j;
            v[j] = i < n ? src[i] : -__builtin_inff();
        }
#pragma unroll
        for (int j = 0; j < PER; j++) key[j] = to_key(v[j]);
    }
    clear_hist(sh);

    // ---- valid count and key range
    {
        uint32_t mn = 0xffffffffu, mx = 0u;
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            if (key[j]) {
                mn = min(mn, key[j]);
                mx = max(mx, key[j]);
                cnt++;
            }
        }
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
        cnt = wave_sum_i32(cnt);
        if (lane == 0) {
            sh.wave_min[wave] = mn;
            sh.wave_max[wave] = mx;
            sh.wave_cnt[wave] = cnt;
        }
    }
    lds_barrier();
    uint32_t lo = 0xffffffffu, hi = 0u;
    int n_valid = 0;
    for (int w = 0; w < kWaves; w++) {
        lo = min(lo, sh.wave_min[w]);
        hi = max(hi, sh.wave_max[w]);
        n_valid += sh.wave_cnt[w];
    }

    uint32_t T;  // select keys > T, plus the first `need` keys == T
    int need;
    if (n_valid <= k) {
        T = 0u;  // every valid key (> 0) is selected
        need = 0;
    } else {
        // invariant: the k-th largest key is in [lo, hi] and kk of the wanted keys are
        // in [lo, hi] (the rest are above hi)
        int kk = k;
        bool resolved = false;
        // ---- first pass in value space: 4096 equal-width bins between the smallest and
        // the largest value.  The bin index is a monotone function of the value, so the
        // bins above the one holding the k-th value hold only selected keys; scores that
        // crowd a few octaves (as logits do) spread over many bins instead of a handful
        // of key-prefix bins.  The few keys of that bin are then ranked by comparison.
        const float vlo = from_key(lo), vhi = from_key(hi);
        const float scale = (float)kBins / (vhi - vlo);
        if (vhi > vlo && __builtin_isfinite(vlo) && __builtin_isfinite(vhi) && __builtin_isfinite(scale)) {
            auto vbin = [&](uint32_t kx) {
                const int b = (int)((from_key(kx) - vlo) * scale);
                return b < kBins - 1 ? b : kBins - 1;
            };
#pragma unroll
            for (int j = 0; j < PER; j++)
                if (key[j] != 0u) atomicAdd(&sh.hist[vbin(key[j])], 1u);
            if (tid == 0) {
                sh.nm = 0;
                sh.blo = 0xffffffffu;
                sh.bhi = 0u;
            }
            lds_barrier();
            {
                int c[kPickPer], bin[kPickPer];
                read_bins_desc(sh.hist, tid, c, bin);
                pick_bin<kThreads, kPickPer>(c, bin, kk, sh.wtot, sh.pick);
            }
            const int d = sh.pick[0];
            const int nd = sh.pick[3];
            kk -= sh.pick[1];  // wanted keys inside bin d, >= 1
            if (nd <= kRankMax) {
#pragma unroll
                for (int j = 0; j < PER; j++) {
                    if (key[j] != 0u && vbin(key[j]) == d) {
                        const int at = atomicAdd(&sh.nm, 1);
                        if (at < kRankMax) {
                            sh.mkey[at] = key[j];
                            sh.midx[at] = tid + kThreads * j;
                        }
                    }
                }
                lds_barrier();
                const int nm = min(sh.nm, kRankMax);
                for (int t = tid; t < nm; t += kThreads) {
                    const uint32_t kt = sh.mkey[t];
                    const int it = sh.midx[t];
                    int gt = 0, rank = 0;
                    for (int u = 0; u < nm; u++) {
                        const uint32_t ku = sh.mkey[u];
                        gt += ku > kt ? 1 : 0;
                        rank += (ku > kt || (ku == kt && sh.midx[u] < it)) ? 1 : 0;
                    }
                    if (rank == kk - 1) {  // the k-th selected key: T and the ties to keep
                        sh.T = kt;
                        sh.need = kk - gt;
                    }
                }
                lds_barrier();
                lo = hi = sh.T;
                kk = sh.need;
                resolved = true;
            } else {
                // many keys in bin d (heavy ties): continue in key space on its key range
#pragma unroll
                for (int j = 0; j < PER; j++) {
                    if (key[j] != 0u && vbin(key[j]) == d) {
                        atomicMin(&sh.blo, key[j]);
                        atomicMax(&sh.bhi, key[j]);
                    }
                }
                lds_barrier();
                lo = sh.blo;
                hi = sh.bhi;
            }
            clear_hist(sh);
            lds_barrier();
        }
        while (!resolved && lo < hi) {
            const uint32_t span_m1 = hi - lo;
            const int bits = 32 - __clz((int)span_m1);
            const int shift = bits > kBinBits ? bits - kBinBits : 0;
#pragma unroll
            for (int j = 0; j < PER; j++) {
                const uint32_t kj = key[j];
                if (kj != 0u && kj >= lo && kj <= hi) atomicAdd(&sh.hist[(kj - lo) >> shift], 1u);
            }
            lds_barrier();
            {
                int c[kPickPer], bin[kPickPer];
                read_bins_desc(sh.hist, tid, c, bin);
                pick_bin<kThreads, kPickPer>(c, bin, kk, sh.wtot, sh.pick);
            }
            const uint32_t dsel = (uint32_t)sh.pick[0];
            kk -= sh.pick[1];
            const uint32_t nlo = lo + (dsel << shift);
            const uint32_t width_m1 = (shift >= 32) ? 0xffffffffu : ((1u << shift) - 1u);
            const uint32_t nhi_raw = nlo + width_m1;
            hi = min(hi, nhi_raw < nlo ? 0xffffffffu : nhi_raw);
            lo = nlo;
            lds_barrier();
            clear_hist(sh);
            lds_barrier();
        }
        T = lo;
        need = kk;  // >= 1 keys equal to T are kept
    }

    // ---- ordered compaction over index order (j, wave, lane); steps past the row's
    // length hold no key and are skipped (their counts are zero)
    const int nsteps = (n + kThreads - 1) / kThreads;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        int cg = 0, ce = 0;
        if (j < nsteps) {
            cg = __popcll(__ballot(key[j] > T));
            ce = __popcll(__ballot(need > 0 && key[j] == T));
        }
        if (lane == 0) {
            sh.cnt_gt[j * kWaves + wave] = cg;
            sh.cnt_eq[j * kWaves + wave] = ce;
        }
    }
    lds_barrier();
    if (wave == 0) {
        // exclusive scans over the kPer * kWaves blocks in index order: ties first (the
        // first `need` ties are kept), then selected = gt + kept ties
        constexpr int E = kPer * kWaves;
        constexpr int per = E / 64;
        int eq[per], gt[per];
        int se = 0;
#pragma unroll
        for (int u = 0; u < per; u++) {
            eq[u] = sh.cnt_eq[lane * per + u];
            gt[u] = sh.cnt_gt[lane * per + u];
            se += eq[u];
        }
        const int ie = wave_incl_scan(se);  // inclusive prefix over lanes
        int tie_before = ie - se;
        int sel[per];
        int ss = 0;
#pragma unroll
        for (int u = 0; u < per; u++) {
            const int take = min(max(need - tie_before, 0), eq[u]);
            sh.off_tie[lane * per + u] = tie_before;
            tie_before += eq[u];
            sel[u] = gt[u] + take;
            ss += sel[u];
        }
        const int is = wave_incl_scan(ss);
        int sel_before = is - ss;
#pragma unroll
        for (int u = 0; u < per; u++) {
            sh.off_sel[lane * per + u] = sel_before;
            sel_before += sel[u];
        }
        if (lane == 63) sh.total = sel_before;
    }
    lds_barrier();
    const int total = sh.total;
    const float* srow = p.scores + (int64_t)row * p.row_stride;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        if (j >= nsteps) continue;
        const int e = j * kWaves + wave;
        const bool is_gt = key[j] > T;
        const bool is_eq = need > 0 && key[j] == T;
        const unsigned long long me = __ballot(is_eq);
        const int tie_rank = sh.off_tie[e] + lanes_below(me);
        const bool sel = is_gt || (is_eq && tie_rank < need);
        const unsigned long long ms = __ballot(sel);
        const int pos = sh.off_sel[e] + lanes_below(ms);
        if (sel) {
            const int c = tid + kThreads * j;
            p.out_idx[(int64_t)row * k + pos] = c;
            if (p.out_vals) p.out_vals[(int64_t)row * k + pos] = srow[c];
        }
    }
    for (int i = total + tid; i < k; i += kThreads) {
        p.out_idx[(int64_t)row * k + i] = -1;
        if (p.out_vals) p.out_vals[(int64_t)row * k + i] = -__builtin_inff();
    }
}

}  // namespace

bool topk_long_rows(int rows, int cols);
size_t topk_long_workspace_bytes(int rows, int cols, int k);
hipError_t launch_topk_long(const TopkParams& p, void* workspace, hipStream_t stream);

size_t topk_workspace_bytes(int rows, int cols, int k) {
    return topk_long_rows(rows, cols) ? topk_long_workspace_bytes(rows, cols, k) : 0;
}

size_t topk_long_zero_bytes(int rows, int cols);
size_t topk_workspace_zero_bytes(int rows, int cols, int k) {
    (void)k;
    return topk_long_rows(rows, cols) ? topk_long_zero_bytes(rows, cols) : 0;
}

// Many rows of at most 32768 columns (prefill): one streaming workgroup per row (see
// topk_stream.hip) keeps the whole chip busy and reads each row once.  Few rows: the
// per-row work is spread over many workgroups (topk_long.hip) or held in LDS here.
bool topk_use_stream(const TopkParams& p) {
    return p.rows >= 512 && p.cols <= kMaxElems && topk_stream_cap(p.cols, p.k) >= 0;
}

hipError_t launch_topk(const TopkParams& p_in, hipStream_t stream) {
    TopkParams p = p_in;
    if (topk_use_stream(p)) return launch_topk_stream(p, stream);
    if (topk_long_rows(p.rows, p.cols)) return launch_topk_long(p, p.workspace, stream);
    hipLaunchKernelGGL(k_topk, dim3(p.rows), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp4idx
