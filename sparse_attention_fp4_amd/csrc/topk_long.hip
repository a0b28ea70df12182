// topk_long.hip -- exact top-k over long score rows (more columns than one workgroup
// holds), spread over many workgroups, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Same order and output as topk.hip (larger first, ties to the smaller column, -inf
// and NaN never selected, result in increasing column order, -1 padded).  Scores map
// to order-preserving 32-bit keys; digit 1 is key bits [31:20], digit 2 bits [19:8].
// A row is cut into chunks of 4096 columns; chunks past a row's end are skipped.
// Rows of at most 13 chunks, when every die can hold its rows' chunk workgroups at once
// (rows r, r + 8, ... on die r % 8), and many rows of at most 8 chunks of 16384
// columns (up to 32 rows, or 48 to 64), run as one kernel whose workgroups wait for each
// other in memory (k_coop, below).  Otherwise workgroups exchange data only across
// kernel boundaries (a device-wide fence inside a kernel costs microseconds on this
// multi-die part), in three kernels:
//   1. hist:    each chunk (a few consecutive chunks when many rows fill the chip)
//               builds the histogram of digit 1 of its keys in LDS and adds its
//               nonzero bins to the row's histogram (global atomics).
//   2. collect: each chunk reads the row's histogram, finds the bin d1 holding the
//               row's k-th largest key, and stores a bitmap of its columns above d1
//               (all selected) with their count, and its keys in d1 (the candidates,
//               with their columns and count).
//   3. finish:  one workgroup per group of up to 8 consecutive chunks (one chunk each
//               when there are few rows).  Each reads the row's candidates (every
//               chunk's first slots in one round of loads; a chunk with more is read
//               again with wider slots, or round by round), the counts and its chunks'
//               bitmaps, finds the digit-2 bin d2 holding the k-th key from an LDS
//               histogram of the candidates, ranks the candidates with prefix (d1, d2)
//               by direct comparison when not all of them are kept (digit passes
//               handle more than 1024 of them), and counts the selected columns of the
//               earlier chunks: that count is where its own chunks' columns go in the
//               output, written in order from popcount scans of their bitmaps.  The
//               first group's workgroup clears the row's histogram for the next call.
// The workspace must be zero-filled before its first use; every call leaves the
// histogram zero-filled again.
#include <algorithm>

#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kChunk = 4096;          // columns per chunk workgroup
// Threads of a histogram or collect workgroup (CT below): 1024 (4 keys a thread) when
// few rows leave most of the chip idle, so each chunk's per-key loops are short
// (4 rows x 100k: top-k 14.6 -> 14.0 us); 512 (8 keys a thread) when many rows fill
// it (64 rows: 27.8 against 32.7 us with 1024).
constexpr int kCTFew = 1024, kCTMany = 512;
constexpr int kBins = 4096;
constexpr int kWords = kChunk / 32;   // bitmap words per chunk
constexpr int kMaxChunks = 128;    // rows of up to 524288 columns
constexpr int kWaveOfGroups = 512;  // workgroups that keep the chip busy (two a CU)

struct RowState {
    int d1;         // digit-1 bin of the k-th largest key, or -1 when every valid key is kept
    int kk;         // wanted keys inside bin d1
};

struct LongWs {
    uint32_t* ctr;       // [rows][64]  one-kernel path: arrivals, wait failed, done (a line of its
                         //             own per row); zero between calls
    RowState* st;        // [rows]
    uint32_t* hist;      // [rows][kBins]            digit 1 of the keys; zero between calls
    uint32_t* bitmap;    // [rows][n_chunks * kWords] columns above bin d1
    uint2* cand;         // [rows][n_chunks][kChunk]  candidates (bin d1): (key, column), column order
    int32_t* cnum;       // [rows][n_chunks]          candidates per chunk
    int32_t* cabove;     // [rows][n_chunks]          columns above bin d1 per chunk
    int n_chunks;
    int cstride;         // candidate slots a chunk (its columns)
    size_t zero_end;     // bytes from the base through hist: zero when a call starts
};

__device__ __forceinline__ uint32_t to_key(float v) {
    if (!(v > -__builtin_inff())) return 0u;
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int row_len(const TopkParams& p, int row) {
    int len = p.cols;
    if (p.row_lens) len = min(max(p.row_lens[row], 0), p.cols);
    return len;
}

// A candidate (key, column) read at device scope: in the one-kernel path other
// workgroups of the same kernel wrote it (device-scope stores, counted before the wait
// that ends).  The three kernels' round-by-round reloads share it (a plain load would
// do there; those reloads are rare).
__device__ __forceinline__ uint2 ld_cand(const uint2* q) {
    const uint64_t x = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<uint2*>(q)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
}

// Thread t of CT holds elements t + CT * j of the chunk (index order = j, wave, lane);
// columns at or past len read as -inf.
template <int CT>
__device__ __forceinline__ void load_chunk_raw(const TopkParams& p, int row, int len, int chunk,
                                               float (&v)[kChunk / CT]) {
    const int c0 = chunk * kChunk;
    const int n = max(0, min(len - c0, kChunk));
    const float* src = p.scores + (int64_t)row * p.row_stride + c0;
#pragma unroll
    for (int j = 0; j < kChunk / CT; j++) {
        const int i = threadIdx.x + CT * j;
        v[j] = i < n ? src[i] : -__builtin_inff();
    }
}

// ---------------------------------------------------------------- 1. hist
// hs: chunks per workgroup (chunks [hg * hs, +hs) of the row, one LDS histogram and one
// flush for all of them); chunks past the row's end are skipped.
template <int CT>
__global__ __launch_bounds__(CT) void k_hist(const TopkParams p, LongWs ws, int hs) {
    constexpr int kP = kChunk / CT;
    __shared__ uint32_t h[kBins];
    const int nhg = (ws.n_chunks + hs - 1) / hs;
    const int row = blockIdx.x / nhg, hg = blockIdx.x - row * nhg;
    if (row >= p.rows) return;
    const int len = row_len(p, row);
    const int c_begin = hg * hs, c_end = min(min(c_begin + hs, ws.n_chunks), (len + kChunk - 1) / kChunk);
    if (c_begin >= c_end) return;  // past the row's end
    for (int i = threadIdx.x; i < kBins; i += CT) h[i] = 0u;
    float v[kP];
    load_chunk_raw<CT>(p, row, len, c_begin, v);
    lds_barrier();
    for (int c = c_begin; c < c_end; c++) {
        uint32_t key[kP];
#pragma unroll
        for (int j = 0; j < kP; j++) key[j] = to_key(v[j]);
        if (c + 1 < c_end) load_chunk_raw<CT>(p, row, len, c + 1, v);  // in flight with the atomics
#pragma unroll
        for (int j = 0; j < kP; j++)
            if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
    }
    lds_barrier();
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += CT)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------- 2. collect
template <int CT>
struct CollectShared {
    static_assert((kChunk / CT) * (CT / 64) == 64, "the collect scan covers 64 (step, wave) blocks");
    int wtot[CT / 64];
    int pick[4];
    int total;
    int wab[CT / 64];                  // columns above d1 of each wave
    alignas(8) uint32_t bits[kWords];
    int cnt[64];
    int off[64];
};

// This thread's bins of the row's histogram, 4095 - (kBins / CT) t down, as 16-byte loads.
template <int CT>
__device__ __forceinline__ void load_hist_bins(const LongWs& ws, int row, uint4 (&hv)[kBins / CT / 4]) {
    const uint4* gh4 = reinterpret_cast<const uint4*>(ws.hist + (int64_t)row * kBins);
#pragma unroll
    for (int i = 0; i < kBins / CT / 4; i++) hv[i] = gh4[kBins / 4 - 1 - (kBins / CT / 4) * threadIdx.x - i];
}

// The bin of the row's k-th largest key from the row's histogram (hv: this thread's
// bins).  Returns d1 (-1 when every valid key is kept) and kk, the keys wanted in d1.
template <int CT>
__device__ __forceinline__ void row_threshold_bin(CollectShared<CT>& sh, const TopkParams& p,
                                                  const uint4 (&hv)[kBins / CT / 4], int& d1, int& kk) {
    constexpr int per = kBins / CT;
    int c[per], bin[per];
    // walked from the top ("before" = larger keys)
#pragma unroll
    for (int i = 0; i < per / 4; i++) {
        c[4 * i] = (int)hv[i].w;
        c[4 * i + 1] = (int)hv[i].z;
        c[4 * i + 2] = (int)hv[i].y;
        c[4 * i + 3] = (int)hv[i].x;
    }
#pragma unroll
    for (int i = 0; i < per; i++) bin[i] = kBins - 1 - (threadIdx.x * per + i);
    pick_bin<CT, per>(c, bin, p.k, sh.wtot, sh.pick);
    if (sh.pick[2] <= p.k) {
        d1 = -1;
        kk = 0;
    } else {
        d1 = sh.pick[0];
        kk = p.k - sh.pick[1];
    }
}

template <int CT>
__global__ __launch_bounds__(CT) void k_collect(const TopkParams p, LongWs ws) {
    constexpr int kP = kChunk / CT;
    __shared__ CollectShared<CT> sh;
    const int nch = ws.n_chunks;
    const int row = blockIdx.x / nch, chunk = blockIdx.x - row * nch;
    if (row >= p.rows) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the row's histogram first (it does not wait for the row's length), then the chunk
    uint4 hv[kBins / CT / 4];
    load_hist_bins<CT>(ws, row, hv);
    const int len = row_len(p, row);
    const int c0 = chunk * kChunk;
    float v[kP];
    load_chunk_raw<CT>(p, row, len, chunk, v);
    // a chunk past the row's end stores nothing (the finish never reads it); the first
    // chunk always runs, since it stores the row's state
    if (chunk > 0 && c0 >= len) return;
    uint32_t key[kP];
#pragma unroll
    for (int j = 0; j < kP; j++) key[j] = to_key(v[j]);
    int d1, kk;
    row_threshold_bin<CT>(sh, p, hv, d1, kk);  // ends with a barrier

    // ---- bitmap of the columns above bin d1 and its count; candidates of bin d1
    bool cand[kP];
    int above = 0;  // this wave's columns above d1 (uniform)
#pragma unroll
    for (int j = 0; j < kP; j++) {
        const uint32_t kj = key[j];
        const int dig = (int)(kj >> 20);
        const bool up = kj != 0u && (d1 < 0 || dig > d1);
        // a wave covers 64 consecutive columns = two bitmap words, from an even word
        const unsigned long long ma = __ballot(up);
        above += __popcll(ma);
        if (lane == 0) *reinterpret_cast<unsigned long long*>(&sh.bits[(threadIdx.x + CT * j) >> 5]) = ma;
        cand[j] = d1 >= 0 && kj != 0u && dig == d1;
        const unsigned long long mc = __ballot(cand[j]);
        if (lane == 0) sh.cnt[j * (CT / 64) + wave] = __popcll(mc);
    }
    if (lane == 0) sh.wab[wave] = above;
    lds_barrier();
    if (wave == 0) {  // exclusive scan over the 64 (step, wave) blocks
        const int x = sh.cnt[lane];
        const int s = wave_incl_scan(x);
        sh.off[lane] = s - x;
        if (lane == 63) sh.total = s;
    }
    lds_barrier();
    // Global writes come last: a barrier after them would wait for their completion.
    uint2* dst = ws.cand + ((int64_t)row * nch + chunk) * kChunk;
#pragma unroll
    for (int j = 0; j < kP; j++) {
        const unsigned long long mc = __ballot(cand[j]);
        if (cand[j]) {
            const int pos = sh.off[j * (CT / 64) + wave] + lanes_below(mc);
            dst[pos] = make_uint2(key[j], (uint32_t)(c0 + threadIdx.x + CT * j));
        }
    }
    uint32_t* gbits = ws.bitmap + (int64_t)row * nch * kWords + chunk * kWords;
    for (int i = threadIdx.x; i < kWords; i += CT) gbits[i] = sh.bits[i];
    if (threadIdx.x == 0) {
        int ab = 0;
#pragma unroll
        for (int w = 0; w < CT / 64; w++) ab += sh.wab[w];
        ws.cnum[(int64_t)row * nch + chunk] = sh.total;
        ws.cabove[(int64_t)row * nch + chunk] = ab;
        if (chunk == 0) {
            ws.st[row].d1 = d1;
            ws.st[row].kk = kk;
        }
    }
}

// ---------------------------------------------------------------- 3. finish
// FT: threads of a finishing workgroup (kCTFew or kCTMany, as for the other passes).
// Its candidate registers hold kSlots candidates, FT / 64 chunks' columns at most
// (one wave writes each).
constexpr int kSlots = 4096;
constexpr int kRankMax = 1024;  // candidates at the threshold prefix ranked by comparison
static_assert(kMaxChunks * 32 == kSlots, "32 up-front candidate slots a chunk or more");

template <int FT>
struct FinishShared {
    static constexpr int kGMax = FT / 64;
    alignas(16) uint32_t h[kBins];     // digit-2 histogram, then the narrowing passes'
    alignas(16) uint32_t bits[kGMax * kWords];  // this workgroup's chunks' bitmaps
    uint32_t mkey[kRankMax];           // candidates with the threshold prefix (d1, d2)
    int mcol[kRankMax];
    int cnum[kMaxChunks];
    int coff[kMaxChunks + 1];          // candidate prefix over chunks (flat mode)
    int wtot[FT / 64];
    int part[2][4];                    // waves 0, 1: columns above d1 before this chunk, in the row;
                                       // candidates, most candidates of one chunk
    int pick[4];
    int ctot[kGMax];                   // selected columns of each of this workgroup's chunks
    int nm;
    int before;                        // selected candidates of earlier chunks
};

// Candidate registers: kSlots / FT per thread.  In the common case they hold every
// candidate of the row (registers 2j and 2j+1 hold slots 2q % spec and 2q % spec + 1 of
// chunk 2q / spec, q = threadIdx.x + FT * j); otherwise ("flat" mode) they hold
// candidates [round * kSlots, +kSlots) of the row in chunk order, reloaded round by
// round.
template <int FT>
struct CandRegs {
    static constexpr int kCR = kSlots / FT;
    static_assert(kCR % 2 == 0, "up-front loads fill the registers in slot pairs");
    uint32_t key[kCR];
    int col[kCR];  // -1: no candidate
};

// Candidate i of the row (flat order) lives in chunk c with coff[c] <= i < coff[c+1].
template <int FT>
__device__ __forceinline__ int64_t cand_slot(const FinishShared<FT>& sh, const LongWs& ws, int row, int nch, int i) {
    int lo = 0, hi = nch;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.coff[mid] <= i) lo = mid;
        else hi = mid;
    }
    return ((int64_t)row * ws.n_chunks + lo) * ws.cstride + (i - sh.coff[lo]);
}

template <int FT>
__device__ __forceinline__ void load_flat(CandRegs<FT>& r, const FinishShared<FT>& sh, const LongWs& ws, int row,
                                          int nch, int m, int round) {
    constexpr int kCR = CandRegs<FT>::kCR;
    uint2 v[kCR];
#pragma unroll
    for (int j = 0; j < kCR; j++) {
        const int i = round * kSlots + threadIdx.x + FT * j;
        v[j] = i < m ? ld_cand(ws.cand + cand_slot(sh, ws, row, nch, i)) : make_uint2(0u, 0xffffffffu);
    }
#pragma unroll
    for (int j = 0; j < kCR; j++) {
        r.key[j] = v[j].x;
        r.col[j] = (int)v[j].y;
    }
}

// One digit pass over the candidates that pass `keep`: histogram of digit(key, col)
// and the bin holding the kk-th element in the given order.
template <int FT, bool FLAT, typename Keep, typename Digit>
__device__ __forceinline__ void cand_pass(FinishShared<FT>& sh, CandRegs<FT>& r, const LongWs& ws, int row, int nch,
                                          int m, int rounds, int kk, bool descending, Keep keep, Digit digit) {
    constexpr int kCR = CandRegs<FT>::kCR;
    for (int i = threadIdx.x; i < kBins; i += FT) sh.h[i] = 0u;
    lds_barrier();
    for (int round = 0; round < rounds; round++) {
        if (FLAT && rounds > 1) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
        for (int j = 0; j < kCR; j++)
            if (r.col[j] >= 0 && keep(r.key[j], r.col[j])) atomicAdd(&sh.h[digit(r.key[j], r.col[j])], 1u);
    }
    lds_barrier();
    constexpr int per = kBins / FT;
    int c[per], bin[per];
#pragma unroll
    for (int b = 0; b < per; b++) {
        bin[b] = descending ? kBins - 1 - (threadIdx.x * per + b) : threadIdx.x * per + b;
        c[b] = (int)sh.h[bin[b]];
    }
    pick_bin<FT, per>(c, bin, kk, sh.wtot, sh.pick);
}

// Marks this workgroup's selected candidates in its bitmaps and adds those of earlier
// chunks to sh.before.  FLAT (some chunk has more candidates than its up-front slots):
// the candidates are read in row order, once when they fit the registers, else again
// in every pass, round by round.  Otherwise registers [0, 2 * jr) hold them all.
// Chunks are 2^LCH columns, with 2^(LCH - 5) bitmap words each.
template <int FT, bool FLAT, int LCH = 12>
__device__ __forceinline__ void select_candidates(FinishShared<FT>& sh, CandRegs<FT>& r, const LongWs& ws, int row,
                                                  int nch, int m, int rounds, int jr, int d1, int kk, int chunk,
                                                  int nown) {
    constexpr int kCR = CandRegs<FT>::kCR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int before = 0;  // this thread's selected candidates of earlier chunks
    if (FLAT && rounds == 1) load_flat(r, sh, ws, row, nch, m, 0);
    // ---- digit 2 of the candidates: LDS histogram and its pick
    for (int round = 0; round < rounds; round++) {
        if (FLAT && rounds > 1) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
        for (int j = 0; j < kCR; j++)
            if (j < 2 * jr && r.col[j] >= 0) atomicAdd(&sh.h[(r.key[j] >> 8) & (kBins - 1)], 1u);
    }
    lds_barrier();
    {
        // thread t owns PB = kBins / FT bins, 4095 - PB t down (16-byte reads), walked from
        // the top: wave totals first, then the thread whose bins hold the kk-th key finds
        // its bin
        constexpr int PB = kBins / FT;
        static_assert(PB % 4 == 0, "whole 16-byte reads");
        const uint4* h4 = reinterpret_cast<const uint4*>(sh.h + (kBins - PB - PB * threadIdx.x));
        int c[PB];
#pragma unroll
        for (int i = 0; i < PB / 4; i++) {
            const uint4 v = h4[PB / 4 - 1 - i];
            c[4 * i] = (int)v.w;
            c[4 * i + 1] = (int)v.z;
            c[4 * i + 2] = (int)v.y;
            c[4 * i + 3] = (int)v.x;
        }
        int s = 0;
#pragma unroll
        for (int b = 0; b < PB; b++) s += c[b];
        const int incl = wave_incl_scan(s);
        if (lane == 63) sh.wtot[wave] = incl;
        lds_barrier();
        // keys in the bins above this thread's: the earlier waves' totals (one LDS read
        // a lane and a wave scan) and this wave's lanes before it
        const int wt = wave_incl_scan(lane < FT / 64 ? (int)sh.wtot[lane] : 0);
        const int uw = __builtin_amdgcn_readfirstlane(wave);
        int ex = incl - s + (uw > 0 ? __builtin_amdgcn_readlane(wt, uw - 1) : 0);
        if (ex < kk && kk <= ex + s) {
#pragma unroll
            for (int b = 0; b < PB; b++) {
                if (ex + c[b] >= kk) {
                    sh.pick[0] = kBins - 1 - PB * threadIdx.x - b;
                    sh.pick[1] = ex;
                    sh.pick[3] = c[b];
                    break;
                }
                ex += c[b];
            }
        }
    }
    lds_barrier();
    const uint32_t preA = ((uint32_t)d1 << 12) | (uint32_t)sh.pick[0];
    kk -= sh.pick[1];                      // keys wanted with prefix preA, >= 1
    const int n_pre = sh.pick[3];          // candidates with prefix preA
    // selected: prefix above preA, or at it and within the first kk of the row's
    // order (larger key, then smaller column): key > T, or key == T and col <= c_cut
    uint32_t T = preA << 8;
    int c_cut = 0x7fffffff;                // every candidate at the prefix when kk == n_pre
    if (__builtin_expect(kk < n_pre && n_pre <= kRankMax, 0)) {
        // ---- the candidates at the prefix go to LDS and are ranked by comparison
        for (int round = 0; round < rounds; round++) {
            if (FLAT && rounds > 1) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
            for (int j = 0; j < kCR; j++) {
                if (j < 2 * jr && r.col[j] >= 0 && (r.key[j] >> 8) == preA) {
                    const int at = atomicAdd(&sh.nm, 1);
                    if (at < kRankMax) {   // n_pre bounds it; the test keeps LDS safe
                        sh.mkey[at] = r.key[j];
                        sh.mcol[at] = r.col[j];
                    }
                }
            }
        }
        lds_barrier();
        const int nm = min(sh.nm, kRankMax);
        // the kk-th of the prefix candidates in the row's order sets (T, c_cut)
        for (int t = threadIdx.x; t < nm; t += FT) {
            const uint32_t kt = sh.mkey[t];
            const int ct = sh.mcol[t];
            int rank = 0;
            for (int u = 0; u < nm; u++) {
                const uint32_t ku = sh.mkey[u];
                rank += (ku > kt || (ku == kt && sh.mcol[u] < ct)) ? 1 : 0;
            }
            if (rank == kk - 1) {
                sh.pick[0] = (int)kt;
                sh.pick[1] = ct;
            }
        }
        lds_barrier();
        T = (uint32_t)sh.pick[0];
        c_cut = sh.pick[1];
    } else if (__builtin_expect(kk < n_pre, 0)) {
        // ---- many candidates share the prefix: digit passes over them
        cand_pass<FT, FLAT>(sh, r, ws, row, nch, m, rounds, kk, true,
                  [&](uint32_t kx, int) { return (kx >> 8) == preA; },
                  [&](uint32_t kx, int) { return (int)(kx & 0xffu); });
        T = (preA << 8) | (uint32_t)sh.pick[0];
        kk -= sh.pick[1];  // ties at T to keep, >= 1
        const int ties = sh.pick[3];
        if (kk < ties) {
            // the kk-th smallest column among the ties at T: bits [30:20], [19:8], [7:0]
            cand_pass<FT, FLAT>(sh, r, ws, row, nch, m, rounds, kk, false, [&](uint32_t kx, int) { return kx == T; },
                      [&](uint32_t, int col) { return (int)(((uint32_t)col >> 20) & 0x7ffu); });
            const uint32_t c1 = (uint32_t)sh.pick[0];
            kk -= sh.pick[1];
            cand_pass<FT, FLAT>(sh, r, ws, row, nch, m, rounds, kk, false,
                      [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 20) == c1; },
                      [&](uint32_t, int col) { return (int)(((uint32_t)col >> 8) & 0xfffu); });
            const uint32_t c2 = (c1 << 12) | (uint32_t)sh.pick[0];
            kk -= sh.pick[1];
            cand_pass<FT, FLAT>(sh, r, ws, row, nch, m, rounds, kk, false,
                      [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 8) == c2; },
                      [&](uint32_t, int col) { return (int)((uint32_t)col & 0xffu); });
            c_cut = (int)((c2 << 8) | (uint32_t)sh.pick[0]);
        }
    }
    // ---- selected candidates: earlier chunks' are counted, this workgroup's marked
    for (int round = 0; round < rounds; round++) {
        if (FLAT && rounds > 1) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
        for (int j = 0; j < kCR; j++) {
            const uint32_t kx = r.key[j];
            const int col = r.col[j];
            if (j >= 2 * jr || col < 0) continue;
            const uint32_t pre = kx >> 8;
            const bool sel = pre > preA || (pre == preA && (kx > T || (kx == T && col <= c_cut)));
            if (!sel) continue;
            const int c = col >> LCH;
            if (c < chunk) before++;
            else if (c < chunk + nown)
                atomicOr(&sh.bits[((c - chunk) << (LCH - 5)) + ((col & ((1 << LCH) - 1)) >> 5)], 1u << (col & 31));
        }
    }
    const int wb = wave_sum_i32(before);
    if (lane == 0 && wb) atomicAdd(&sh.before, wb);
    lds_barrier();
}

// gsz: chunks per workgroup (1..FT / 64); chunks [grp * gsz, +gsz) of the row.
template <int FT>
__global__ __launch_bounds__(FT) void k_finish(const TopkParams p, LongWs ws, int gsz) {
    constexpr int kCR = CandRegs<FT>::kCR, kGMax = FT / 64;
    __shared__ FinishShared<FT> sh;
    const int nch = ws.n_chunks;
    const int ngrp = (nch + gsz - 1) / gsz;
    const int row = blockIdx.x / ngrp, grp = blockIdx.x - row * ngrp;
    if (row >= p.rows) return;
    const int chunk = grp * gsz;  // first chunk
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int k = p.k;
    const int64_t rc = (int64_t)row * nch;
    // candidate slots read per chunk up front: 2048 / nch rounded down to a power of two,
    // from 32 (128 chunks fill the registers) to 256 (few chunks cost few loads)
    int lspec = 5;
    while (lspec < 8 && (nch << (lspec + 1)) <= 2048) lspec++;
    const int spec = 1 << lspec;
    // slot-pair registers that can hold a candidate up front (the rest stay empty)
    const int jn = min(kCR / 2, (nch * spec / 2 + FT - 1) / FT);

    // ---- one round of loads: state, counts, these chunks' bitmaps and the first `spec`
    // candidate slots of every chunk (read before the counts are known; slots past a
    // count are ignored), 16 bytes per lane where the arrays allow
    if (grp == 0) {  // the digit-1 histogram was last read by the collect pass: clear it
        uint4* gh = reinterpret_cast<uint4*>(ws.hist + (int64_t)row * kBins);
        for (int i = threadIdx.x; i < kBins / 4; i += FT) gh[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const int d1 = ws.st[row].d1;
    int kk = ws.st[row].kk;
    // everything is loaded for all nch chunks and masked once the row's length is in:
    // the collect pass wrote nothing for chunks past the row's end (ncr: chunks in use)
    const int len = row_len(p, row);
    int my_cnum = threadIdx.x < nch ? ws.cnum[rc + threadIdx.x] : 0;
    int my_above = threadIdx.x < nch ? ws.cabove[rc + threadIdx.x] : 0;
    static_assert(kGMax * kWords / 4 <= FT, "one 16-byte bitmap load per thread at most");
    uint4 bw = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < min(gsz, nch - chunk) * (kWords / 4))
        bw = reinterpret_cast<const uint4*>(ws.bitmap + (rc + chunk) * kWords)[threadIdx.x];
    uint4 sv[kCR / 2];
#pragma unroll
    for (int j = 0; j < kCR / 2; j++) {
        const int q = threadIdx.x + FT * j;
        const int c = (2 * q) >> lspec, slot = (2 * q) & (spec - 1);
        sv[j] = j < jn && c < nch ? *reinterpret_cast<const uint4*>(ws.cand + (rc + c) * kChunk + slot)
                                  : make_uint4(0u, 0xffffffffu, 0u, 0xffffffffu);
    }
    // LDS set-up while the loads are in flight
    const int ncr = max(1, (len + kChunk - 1) / kChunk);
    if (chunk >= ncr) return;  // only chunks past the row's end
    const int nown = min(gsz, ncr - chunk);  // chunks this workgroup writes
    if (threadIdx.x >= ncr) my_cnum = my_above = 0;
    if (threadIdx.x >= nown * (kWords / 4)) bw = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kBins / 4 / FT; i++) reinterpret_cast<uint4*>(sh.h)[threadIdx.x + FT * i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) {
        sh.nm = 0;
        sh.before = 0;
    }
    static_assert(kMaxChunks <= 128, "per-chunk counts fit waves 0 and 1");
    if (wave < 2) {  // sums over chunks: threads 0..127 hold one chunk each
        const int ab = wave_sum_i32(threadIdx.x < chunk ? my_above : 0);
        const int at = wave_sum_i32(my_above);
        const int cs = wave_incl_scan(my_cnum);
        if (threadIdx.x < nch) sh.coff[threadIdx.x + 1] = cs;  // this wave's part; wave 1 adds wave 0's below
        if (lane == 0) {
            sh.part[wave][0] = ab;
            sh.part[wave][1] = at;
        }
        if (lane == 63) sh.part[wave][2] = cs;
        const int mx = (int)wave_max_u32((uint32_t)my_cnum);
        if (lane == 0) sh.part[wave][3] = mx;
    }
    if (threadIdx.x < nch) sh.cnum[threadIdx.x] = my_cnum;
    if (threadIdx.x < kGMax * kWords / 4) reinterpret_cast<uint4*>(sh.bits)[threadIdx.x] = bw;
    bool flat = __syncthreads_or(my_cnum > spec) != 0;
    const int above_before = sh.part[0][0] + sh.part[1][0];
    const int above_total = sh.part[0][1] + sh.part[1][1];
    const int m = sh.part[0][2] + sh.part[1][2];  // candidates of the row
    int rounds = 1;                               // reload rounds
    int ls = lspec, jr = jn;                      // slots a chunk (log2), pair registers in use
    if (flat) {
        // some chunk has more candidates than its up-front slots: when wider slots still
        // fit every chunk in the registers, one more round of loads reads them that way
        const int cmax = max(sh.part[0][3], sh.part[1][3]);
        int lw = lspec + 1;
        while ((1 << lw) < cmax) lw++;
        if ((nch << lw) <= kSlots) {
            ls = lw;
            jr = min(kCR / 2, ((nch << lw) / 2 + FT - 1) / FT);
#pragma unroll
            for (int j = 0; j < kCR / 2; j++) {
                const int q = threadIdx.x + FT * j;
                const int c = (2 * q) >> ls, slot = (2 * q) & ((1 << ls) - 1);
                sv[j] = j < jr && c < nch ? *reinterpret_cast<const uint4*>(ws.cand + (rc + c) * kChunk + slot)
                                          : make_uint4(0u, 0xffffffffu, 0u, 0xffffffffu);
            }
            flat = false;
        }
    }
    CandRegs<FT> r;
    if (flat) {
        // chunk-order prefix of the candidate counts for the flat reloads
        if (threadIdx.x == 0) sh.coff[0] = 0;
        if (threadIdx.x >= 64 && threadIdx.x < nch) sh.coff[threadIdx.x + 1] += sh.part[0][2];
        lds_barrier();
        rounds = (m + kSlots - 1) / kSlots;
    } else {
#pragma unroll
        for (int j = 0; j < kCR / 2; j++) {
            const int q = threadIdx.x + FT * j;
            const int c = (2 * q) >> ls, slot = (2 * q) & ((1 << ls) - 1);
            const int cn = c < nch ? sh.cnum[c] : 0;
            r.key[2 * j] = sv[j].x;
            r.col[2 * j] = slot < cn ? (int)sv[j].y : -1;
            r.key[2 * j + 1] = sv[j].z;
            r.col[2 * j + 1] = slot + 1 < cn ? (int)sv[j].w : -1;
        }
    }

    if (d1 >= 0) {
        if (__builtin_expect(flat, 0))
            select_candidates<FT, true>(sh, r, ws, row, nch, m, rounds, kCR / 2, d1, kk, chunk, nown);
        else
            select_candidates<FT, false>(sh, r, ws, row, nch, m, 1, jr, d1, kk, chunk, nown);
    }

    // ---- the chunks' columns in order: wave w writes chunk chunk + w, lane l its
    // bitmap words 2l and 2l+1
    static_assert(kWords == 128, "two bitmap words per lane of one wave");
    const uint32_t w0 = sh.bits[wave * kWords + 2 * lane], w1 = sh.bits[wave * kWords + 2 * lane + 1];
    const int cnt = __popc(w0) + __popc(w1);
    const int incl = wave_incl_scan(cnt);
    if (gsz > 1) {
        if (lane == 63) sh.ctot[wave] = incl;
        lds_barrier();
    }
    if (wave < nown) {
        int base = above_before + sh.before;
        for (int w = 0; w < wave; w++) base += sh.ctot[w];
        int pos = base + incl - cnt;
        const float* srow = p.scores + (int64_t)row * p.row_stride;
        int32_t* oidx = p.out_idx + (int64_t)row * k;
        float* oval = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
        const int cbase = (chunk + wave) * kChunk + 64 * lane;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t bits = h ? w1 : w0;
            while (bits && pos < k) {
                const int col = cbase + 32 * h + __ffs((int)bits) - 1;
                oidx[pos] = col;
                if (oval) oval[pos] = srow[col];
                pos++;
                bits &= bits - 1u;
            }
        }
    }
    // every valid key kept (fewer than k): the workgroup of the row's last chunk pads it
    if (d1 < 0 && chunk + nown == ncr) {
        int32_t* oidx = p.out_idx + (int64_t)row * k;
        float* oval = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
        for (int i = min(above_total, k) + threadIdx.x; i < k; i += FT) {
            oidx[i] = -1;
            if (oval) oval[i] = -__builtin_inff();
        }
    }
}

// ---------------------------------------------------------------- one kernel for few rows
// Rows r, r + 8, ... share die r % 8 and all their chunk workgroups run at once there
// (the dispatcher deals block b to die b % 8; each die has 32 CUs); a row's chunks
// meet at two waits in memory instead of two kernel boundaries: a wait costs about 0.6
// us among the workgroups of one die (1.1 us across dies), a boundary about 2 us plus
// slow first loads of what the previous kernel wrote.  All exchange goes through device-scope
// atomics, loads and stores, so the result does not depend on the placement, only the
// speed does.  Each row's counters sit on a 256-byte line of their own (sharing one
// line between rows made each wait about 1.5 us).
//   1. each chunk (1024 V columns, V keys a thread, kept in registers) adds the
//      digit-1 histogram of its keys to the row's; wait for the row's chunks;
//   2. each chunk finds d1 and kk from the row's histogram, keeps the bitmap of its
//      columns above d1 in LDS, stores its candidates (keys in d1) and both counts;
//      wait;
//   3. each chunk reads every candidate of the row, selects as the finishing pass
//      does, and writes its own columns in order.
// A wait is bounded (g_wait_limit polls); when one runs out, the row is marked and the
// last of its workgroups to end recomputes it alone from the scores.  That workgroup
// (the last to end, failed or not) also clears the row's counters and histogram.
constexpr int kCoopMaxW = 13;   // chunk workgroups a row (see coop_shape for the crossover)
constexpr int kCoopDieWG = 32;  // chunk workgroups a die holds at once (one a CU)
constexpr int kCoopMaxW16 = 8;  // chunk workgroups a row with 16 keys a thread
constexpr int kCoopRowsMin16 = 48;  // fewest rows that take 16 keys a thread two a CU
constexpr int kSc1 = 16;        // cache-policy bit of a device-scope buffer access
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct CoopShared {
    FinishShared<1024> f;
    int ok;
    int wcand[16];   // candidates of each wave
    int wabove[16];  // columns above d1 of each wave
};

// Counts this workgroup's arrival on the row's counter and waits (bounded) until
// `target` arrivals are in.  Every wave first waits for its own global stores and
// atomics, so what the workgroup wrote is in place before it is counted.  Returns
// false (the same in every thread) when the wait ran out or another workgroup's did.
__device__ __forceinline__ bool coop_wait(uint32_t* ctr, uint32_t target, int limit, int& flag) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1;
        for (int it = 0;; it++) {
            const uint64_t st = __hip_atomic_load(reinterpret_cast<uint64_t*>(ctr), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(st >> 32) != 0u) { ok = 0; break; }
            if ((uint32_t)st >= target) break;
            if (it >= limit) {
                __hip_atomic_fetch_or(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        flag = ok;
    }
    __syncthreads();
    return flag != 0;
}

// The row's exact top-k by one workgroup from the scores alone: three digit passes
// find the k-th key T and how many keys equal to it are kept, then one pass in column
// order writes the selected columns (keys above T, and the first of those equal to T).
__device__ void coop_row_alone(const TopkParams& p, int row, int len, FinishShared<1024>& sh) {
    constexpr int FT = 1024, per = kBins / FT;
    const float* srow = p.scores + (int64_t)row * p.row_stride;
    const int k = p.k;
    auto pass = [&](auto keep, auto digit, int kk) {
        for (int i = threadIdx.x; i < kBins; i += FT) sh.h[i] = 0u;
        lds_barrier();
        for (int i = threadIdx.x; i < len; i += FT) {
            const uint32_t key = to_key(srow[i]);
            if (key && keep(key)) atomicAdd(&sh.h[digit(key)], 1u);
        }
        lds_barrier();
        int c[per], bin[per];
#pragma unroll
        for (int b = 0; b < per; b++) {
            bin[b] = kBins - 1 - (threadIdx.x * per + b);
            c[b] = (int)sh.h[bin[b]];
        }
        pick_bin<FT, per>(c, bin, kk, sh.wtot, sh.pick);
    };
    int kk = k;
    pass([](uint32_t) { return true; }, [](uint32_t x) { return (int)(x >> 20); }, kk);
    uint32_t T = 0u;  // keys above T are kept; of those equal to T, the first take_eq
    int take_eq = 0;
    if (sh.pick[2] > kk) {
        const uint32_t d1 = (uint32_t)sh.pick[0];
        kk -= sh.pick[1];
        pass([&](uint32_t x) { return (x >> 20) == d1; }, [](uint32_t x) { return (int)((x >> 8) & 0xfffu); }, kk);
        const uint32_t pre = (d1 << 12) | (uint32_t)sh.pick[0];
        kk -= sh.pick[1];
        pass([&](uint32_t x) { return (x >> 8) == pre; }, [](uint32_t x) { return (int)(x & 0xffu); }, kk);
        T = (pre << 8) | (uint32_t)sh.pick[0];
        take_eq = kk - sh.pick[1];
    }
    int32_t* oidx = p.out_idx + (int64_t)row * k;
    float* oval = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
    int n_sel = 0, n_eq = 0;
    for (int c0 = 0; c0 < len && n_sel < k; c0 += FT) {
        const int i = c0 + threadIdx.x;
        const float v = i < len ? srow[i] : -__builtin_inff();
        const uint32_t key = to_key(v);
        const bool eq = T != 0u && key == T;
        int ex, tot;
        block_excl_scan<FT>(eq ? 1 : 0, sh.wtot, ex, tot);
        const bool sel = key > T || (eq && n_eq + ex < take_eq);
        int exs, tots;
        block_excl_scan<FT>(sel ? 1 : 0, sh.wtot, exs, tots);
        const int pos = n_sel + exs;
        if (sel && pos < k) {
            oidx[pos] = i;
            if (oval) oval[pos] = v;
        }
        n_sel += tots;
        n_eq += tot;
    }
    for (int i = min(n_sel, k) + (int)threadIdx.x; i < k; i += FT) {
        oidx[i] = -1;
        if (oval) oval[i] = -__builtin_inff();
    }
}

// V: keys a thread (chunks of 1024 V columns); W: chunk workgroups a row; rpd: rows a
// die.  Grid: 8 * rpd * W blocks; block b serves row (b >> 3) / W * 8 + b % 8, chunk
// (b >> 3) % W.
template <int V>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(V == 16 ? 8 : 1, 8))) void k_coop(const TopkParams p, LongWs ws, int W, int rpd, int limit) {
    constexpr int FT = 1024, C = FT * V, CW = C / 32;
    constexpr int LCH = V == 4 ? 12 : V == 8 ? 13 : 14;
    static_assert(V == 4 || V == 8 || V == 16, "4, 8 or 16 keys a thread");
    static_assert(kCoopMaxW <= kCoopDieWG, "every chunk workgroup of a die resident at once");
    static_assert(C == (1 << LCH) && CW <= 16 * kWords, "chunk bitmap fits the finishing LDS");
    constexpr int kCR = CandRegs<FT>::kCR;
    __shared__ CoopShared cs;
    FinishShared<FT>& sh = cs.f;
    const int die = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int lr = rest / W, m = rest - lr * W;
    const int row = lr * 8 + die;
    if (lr >= rpd || row >= p.rows) return;
    const int len = row_len(p, row);
    const int wr = max(1, (len + C - 1) / C);  // chunks in use
    if (m >= wr) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int k = p.k;
    uint32_t* ctr = ws.ctr + (int64_t)row * 64;
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    const int c0 = m * C;
    const float* srow = p.scores + (int64_t)row * p.row_stride;

    // ---- 1. the chunk's digit-1 histogram, added to the row's
    reinterpret_cast<uint4*>(sh.h)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    static_assert(kBins == 4 * FT, "one 16-byte clear a thread");
    if (threadIdx.x == 0) {
        sh.nm = 0;
        sh.before = 0;
    }
    uint32_t key[V];
    {
        const int n = min(len - c0, C);
        float v[V];
#pragma unroll
        for (int j = 0; j < V; j++) {
            const int i = threadIdx.x + FT * j;
            v[j] = i < n ? srow[c0 + i] : -__builtin_inff();
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < V; j++) {
            key[j] = to_key(v[j]);
            if (key[j]) atomicAdd(&sh.h[key[j] >> 20], 1u);
        }
    }
    lds_barrier();
    // consecutive lanes add consecutive bins: one instruction's atomics touch two lines
#pragma unroll
    for (int i = 0; i < kBins / FT; i++) {
        const uint32_t x = sh.h[threadIdx.x + FT * i];
        if (x) __hip_atomic_fetch_add(gh + threadIdx.x + FT * i, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool ok = coop_wait(ctr, (uint32_t)wr, limit, cs.ok);

    if (ok) {
        // ---- 2. d1 and kk from the row's histogram (thread t: bins 4095 - 4t down)
        const v4u hv = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(gh, kBins * 4),
                                                             (kBins / 4 - 1 - (int)threadIdx.x) * 16, 0, kSc1);
        int d1, kk;
        {
            int c[4] = {(int)hv.w, (int)hv.z, (int)hv.y, (int)hv.x}, bin[4];
#pragma unroll
            for (int i = 0; i < 4; i++) bin[i] = kBins - 1 - (4 * (int)threadIdx.x + i);
            pick_bin<FT, 4>(c, bin, k, sh.wtot, sh.pick);
            if (sh.pick[2] <= k) {
                d1 = -1;
                kk = 0;
            } else {
                d1 = sh.pick[0];
                kk = k - sh.pick[1];
            }
        }
        // bitmap of the columns above d1 (LDS) and the candidates in d1 (memory)
        uint2* dst = ws.cand + ((int64_t)row * ws.n_chunks + m) * ws.cstride;
        int above = 0, ncw = 0;  // this wave's columns above d1 and candidates (uniform)
        unsigned long long mc[V];
#pragma unroll
        for (int j = 0; j < V; j++) {
            const uint32_t kj = key[j];
            const int dig = (int)(kj >> 20);
            const bool up = kj != 0u && (d1 < 0 || dig > d1);
            // a wave covers 64 consecutive columns = two bitmap words, from an even word
            const unsigned long long ma = __ballot(up);
            above += __popcll(ma);
            if (lane == 0) *reinterpret_cast<unsigned long long*>(&sh.bits[(threadIdx.x + FT * j) >> 5]) = ma;
            mc[j] = __ballot(d1 >= 0 && kj != 0u && dig == d1);
            ncw += __popcll(mc[j]);
        }
        // the waves' counts, then every wave's offset from one scan of them (no atomics on
        // a shared counter); candidates are stored in (wave, step, lane) order
        if (lane == 0) {
            cs.wcand[wave] = ncw;
            cs.wabove[wave] = above;
        }
        lds_barrier();
        static_assert(FT / 64 <= 16, "wave counts fit one scan");
        const int wsc = wave_incl_scan(lane < FT / 64 ? cs.wcand[lane] : 0);
        const int uw = __builtin_amdgcn_readfirstlane(wave);
        int base = uw > 0 ? __builtin_amdgcn_readlane(wsc, uw - 1) : 0;
        if (ncw) {
#pragma unroll
            for (int j = 0; j < V; j++) {
                if ((mc[j] >> lane) & 1ull) {
                    const uint64_t e = (uint64_t)key[j] | ((uint64_t)(uint32_t)(c0 + threadIdx.x + FT * j) << 32);
                    __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + base + lanes_below(mc[j])), e, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                base += __popcll(mc[j]);
            }
        }
        if (threadIdx.x == 0) {
            const int ntot = __builtin_amdgcn_readlane(wsc, FT / 64 - 1);
            int atot = 0;
#pragma unroll
            for (int w = 0; w < FT / 64; w++) atot += cs.wabove[w];
            __hip_atomic_store(reinterpret_cast<uint32_t*>(ws.cnum) + (int64_t)row * ws.n_chunks + m, (uint32_t)ntot,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(reinterpret_cast<uint32_t*>(ws.cabove) + (int64_t)row * ws.n_chunks + m, (uint32_t)atot,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ok = coop_wait(ctr, 2u * (uint32_t)wr, limit, cs.ok);

        if (ok) {
            // ---- 3. every candidate of the row, then the selection
            const int nch = wr;
            const int64_t rc = (int64_t)row * ws.n_chunks;
            // up-front slots a chunk: kSlots / nch rounded down to a power of two
            int lspec = 5;
            while (lspec < LCH && (nch << (lspec + 1)) <= kSlots) lspec++;
            const int spec = 1 << lspec;
            const int jn = min(kCR / 2, (nch * spec / 2 + FT - 1) / FT);
            const __amdgpu_buffer_rsrc_t cr = make_rsrc(ws.cand + rc * ws.cstride, (uint32_t)(nch * ws.cstride * 8));
            int my_cnum = 0, my_above = 0;
            if (threadIdx.x < nch) {
                my_cnum = (int)__hip_atomic_load(reinterpret_cast<uint32_t*>(ws.cnum) + rc + threadIdx.x, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                my_above = (int)__hip_atomic_load(reinterpret_cast<uint32_t*>(ws.cabove) + rc + threadIdx.x,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            v4u sv[kCR / 2];
#pragma unroll
            for (int j = 0; j < kCR / 2; j++) {
                const int q = threadIdx.x + FT * j;
                const int c = (2 * q) >> lspec, slot = (2 * q) & (spec - 1);
                sv[j] = j < jn && c < nch ? __builtin_amdgcn_raw_buffer_load_b128(cr, (c * ws.cstride + slot) * 8, 0, kSc1)
                                          : v4u{0u, 0xffffffffu, 0u, 0xffffffffu};
            }
            reinterpret_cast<uint4*>(sh.h)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
            static_assert(kCoopMaxW <= 64, "per-chunk counts fit wave 0");
            if (wave == 0) {
                const int ab = wave_sum_i32(lane < m ? my_above : 0);
                const int at = wave_sum_i32(my_above);
                const int cs_ = wave_incl_scan(my_cnum);
                if (lane < nch) sh.coff[lane + 1] = cs_;
                if (lane == 0) {
                    sh.coff[0] = 0;
                    sh.part[0][0] = ab;
                    sh.part[0][1] = at;
                }
                if (lane == 63) sh.part[0][2] = cs_;
                const int mx = (int)wave_max_u32((uint32_t)my_cnum);
                if (lane == 0) sh.part[0][3] = mx;
                if (lane < nch) sh.cnum[lane] = my_cnum;
            }
            bool flat = __syncthreads_or(my_cnum > spec) != 0;
            const int above_before = sh.part[0][0], above_total = sh.part[0][1];
            const int mtot = sh.part[0][2];
            int ls = lspec, jr = jn, rounds = 1;
            if (flat) {
                // some chunk has more candidates than its up-front slots: wider slots when
                // every chunk still fits the registers, else round-by-round reloads
                const int cmax = sh.part[0][3];
                int lw = lspec + 1;
                while ((1 << lw) < cmax) lw++;
                if ((nch << lw) <= kSlots) {
                    ls = lw;
                    jr = min(kCR / 2, ((nch << lw) / 2 + FT - 1) / FT);
#pragma unroll
                    for (int j = 0; j < kCR / 2; j++) {
                        const int q = threadIdx.x + FT * j;
                        const int c = (2 * q) >> ls, slot = (2 * q) & ((1 << ls) - 1);
                        sv[j] = j < jr && c < nch ? __builtin_amdgcn_raw_buffer_load_b128(cr, (c * ws.cstride + slot) * 8, 0, kSc1)
                                                  : v4u{0u, 0xffffffffu, 0u, 0xffffffffu};
                    }
                    flat = false;
                } else {
                    rounds = (mtot + kSlots - 1) / kSlots;
                }
            }
            CandRegs<FT> r;
            if (!flat) {
#pragma unroll
                for (int j = 0; j < kCR / 2; j++) {
                    const int q = threadIdx.x + FT * j;
                    const int c = (2 * q) >> ls, slot = (2 * q) & ((1 << ls) - 1);
                    const int cn = c < nch ? sh.cnum[c] : 0;
                    r.key[2 * j] = sv[j].x;
                    r.col[2 * j] = slot < cn ? (int)sv[j].y : -1;
                    r.key[2 * j + 1] = sv[j].z;
                    r.col[2 * j + 1] = slot + 1 < cn ? (int)sv[j].w : -1;
                }
            }
            if (d1 >= 0) {
                if (__builtin_expect(flat, 0))
                    select_candidates<FT, true, LCH>(sh, r, ws, row, nch, mtot, rounds, kCR / 2, d1, kk, m, 1);
                else
                    select_candidates<FT, false, LCH>(sh, r, ws, row, nch, mtot, 1, jr, d1, kk, m, 1);
            }
            // ---- this chunk's columns in order: thread t holds bitmap word t
            const uint32_t wv = threadIdx.x < CW ? sh.bits[threadIdx.x] : 0u;
            int ex, tot;
            block_excl_scan<FT>(__popc(wv), sh.wtot, ex, tot);
            int pos = above_before + sh.before + ex;
            int32_t* oidx = p.out_idx + (int64_t)row * k;
            float* oval = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
            uint32_t bits = wv;
            while (bits && pos < k) {
                const int col = c0 + 32 * (int)threadIdx.x + __ffs((int)bits) - 1;
                oidx[pos] = col;
                if (oval) oval[pos] = srow[col];
                pos++;
                bits &= bits - 1u;
            }
            // every valid key kept (fewer than k): the row's last chunk pads it
            if (d1 < 0 && m == wr - 1) {
                for (int i = min(above_total, k) + (int)threadIdx.x; i < k; i += FT) {
                    oidx[i] = -1;
                    if (oval) oval[i] = -__builtin_inff();
                }
            }
        }
    }

    // ---- the end: the row's last workgroup recomputes it when a wait ran out, then
    // clears the row's histogram and counters for the next call
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ctr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int last = 0;
        if (old == (uint32_t)(wr - 1)) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            last = __hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ? 2 : 1;
        }
        cs.ok = last;
    }
    __syncthreads();
    const int last = cs.ok;
    if (last) {
        if (last == 2) coop_row_alone(p, row, len, sh);
        __builtin_amdgcn_raw_buffer_store_b128(v4u{0u, 0u, 0u, 0u}, make_rsrc(gh, kBins * 4), (int)threadIdx.x * 16, 0, kSc1);
        if (threadIdx.x < 3) __hip_atomic_store(ctr + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Keys a thread, and chunk workgroups a row, for the one-kernel path, or false when it
// does not apply: rows of more than kCoopMaxW chunks, or more rows a die (rows 8 apart
// share one) than its CUs hold with their chunks.  Its
// in-kernel time grows with the chunks a row (more adds on each histogram bin, more
// candidates to read), while the three kernels' does not: a step of 4 rows (scorer +
// top-k) took 17.1 against 18.7 us at 16384 and 32768 columns (4 and 8 chunks), 17.8
// against 18.7 at 50000 (13), 18.7 against 18.8 at 65536 (16; the top-k alone on
// random rows 13.3 against 12.9, and 13.9 against 13.1 with 8 rows), and 19.5-20.6
// against 19.5 at 100k (25).
// Many rows (more 4096-column chunks than kWaveOfGroups, up to 64 rows of up to 131072
// columns) take 16 keys a thread instead: chunks of 16384 columns, one workgroup a CU
// when a die's rows fit that (up to 32 rows of 131072), else two (55 VGPRs and 34 KB
// of LDS allow it), which pays from 48 rows on.  The top-k alone on full rows against
// the three kernels: one a CU, 20 x 131072 18.1 vs 18.5 us, 32 x 131072 19.3 vs 21.1,
// 32 x 100000 18.6 vs 19.9, 24 x 100000 18.1 vs 18.3; two a CU, 64 x 131072 26.1 vs
// 30.3, 48 x 131072 24.6 vs 25.9, 64 x 100000 24.7 vs 27.2, but 40 x 131072 24.1 vs
// 24.2 and 40 x 100000 23.0 vs 21.1 (unevenly doubled CUs).  Few rows stay with the
// three kernels (4 x 100k: 16.2 vs 13.7 us in one kernel).
// per_cu: the one-kernel workgroups a CU holds at once.
bool coop_shape(int rows, int cols, int& V, int& W, int& per_cu) {
    if (rows < 1) return false;
    const int64_t rpd = (rows + 7) / 8;
    V = 4;
    per_cu = 1;
    W = (cols + 1024 * V - 1) / (1024 * V);
    if (W <= kCoopMaxW && rpd * W <= kCoopDieWG) return true;
    if ((int64_t)rows * ((cols + kChunk - 1) / kChunk) <= kWaveOfGroups) return false;
    V = 16;
    W = (cols + 1024 * V - 1) / (1024 * V);
    per_cu = rpd * W <= kCoopDieWG ? 1 : 2;
    if (per_cu == 2 && rows < kCoopRowsMin16) return false;
    return W <= kCoopMaxW16 && rpd * W <= 2 * kCoopDieWG;
}

int g_wait_limit = 1 << 16;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The three-kernel view of the workspace; the one-kernel path (coop_shape) uses the
// same regions with its own chunk count and candidate stride, so the candidate and
// count regions are sized for both.
LongWs carve(void* base, int rows, int cols, size_t* bytes) {
    LongWs w{};
    w.n_chunks = (cols + kChunk - 1) / kChunk;
    w.cstride = kChunk;
    const size_t rc = (size_t)rows * w.n_chunks;
    size_t cand_row = (size_t)w.n_chunks * kChunk, cnt_row = (size_t)w.n_chunks;
    int cv = 0, cw = 0, cpc = 0;
    if (coop_shape(rows, cols, cv, cw, cpc)) {
        cand_row = std::max(cand_row, (size_t)cw * 1024 * cv);
        cnt_row = std::max(cnt_row, (size_t)cw);
    }
    unsigned char* b = reinterpret_cast<unsigned char*>(base);
    size_t o = 0;
    w.ctr = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + (size_t)rows * 64 * 4);
    w.st = reinterpret_cast<RowState*>(b + o);
    o = align256(o + (size_t)rows * sizeof(RowState));
    w.hist = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + (size_t)rows * kBins * 4);
    w.zero_end = o;
    w.bitmap = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + rc * kWords * 4);
    w.cand = reinterpret_cast<uint2*>(b + o);
    o = align256(o + (size_t)rows * cand_row * sizeof(uint2));
    w.cnum = reinterpret_cast<int32_t*>(b + o);
    o = align256(o + (size_t)rows * cnt_row * 4);
    w.cabove = reinterpret_cast<int32_t*>(b + o);
    o = align256(o + (size_t)rows * cnt_row * 4);
    if (bytes) *bytes = o;
    return w;
}

}  // namespace

// Rows longer than one workgroup holds go here; so do rows of more than 8192 columns
// when there are few of them: spread over chunk workgroups they finish sooner than with
// one workgroup per row (4 rows of 16384 columns: 14.5 against 16.5 us), while many
// rows keep the chip busy one workgroup each.
bool topk_long_rows(int rows, int cols) { return cols > 32768 || (cols > 8192 && rows <= 64); }

// Leading workspace bytes that must be zero when a call starts: the one-kernel path's
// counters, the row states and the histogram come first in the layout (a caller that cannot keep the workspace
// between calls clears just these).
size_t topk_long_zero_bytes(int rows, int cols) { return carve(nullptr, rows, cols, nullptr).zero_end; }

size_t topk_long_workspace_bytes(int rows, int cols, int k) {
    (void)k;
    size_t bytes = 0;
    carve(nullptr, rows, cols, &bytes);
    return bytes;
}

// Compute units of the current device (read once per device): the one-kernel path
// needs all its workgroups resident at once, one a CU.
static int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
    }
    return cus[dev];
}

int set_topk_wait_limit(int polls) {
    const int prev = g_wait_limit;
    if (polls >= 0) g_wait_limit = polls;
    return prev;
}

hipError_t launch_topk_long(const TopkParams& p, void* workspace, hipStream_t stream) {
    LongWs w = carve(workspace, p.rows, p.cols, nullptr);
    if (w.n_chunks > kMaxChunks) return hipErrorInvalidValue;
    int cv = 0, cw = 0, cpc = 0;
    if (coop_shape(p.rows, p.cols, cv, cw, cpc) && 8 * ((p.rows + 7) / 8) * cw <= cpc * device_cus()) {
        // one kernel: every row's chunk workgroups on one die, all resident at once (a
        // device with fewer CUs than the grid, e.g. one die of a partitioned GPU, takes
        // the three kernels instead of waiting on workgroups that cannot start)
        LongWs c = w;
        c.n_chunks = cw;
        c.cstride = 1024 * cv;
        const int rpd = (p.rows + 7) / 8;
        const dim3 grid((unsigned)(8 * rpd * cw));
        if (cv == 4) hipLaunchKernelGGL(k_coop<4>, grid, dim3(1024), 0, stream, p, c, cw, rpd, g_wait_limit);
        else hipLaunchKernelGGL(k_coop<16>, grid, dim3(1024), 0, stream, p, c, cw, rpd, g_wait_limit);
        return hipGetLastError();
    }
    // Few rows: one workgroup per chunk keeps each one short, with 1024 lanes.  Many
    // rows: 512 lanes; the histogram pass takes up to kHMax chunks per workgroup (fewer
    // global atomics on each row's histogram; 64 rows of 32 chunks: 7.8 us with two
    // chunks, 8.1 with four, 8.4 with one) and the finish up to 8, so that the redundant
    // reading and ranking of each row's candidates stays near one pass over the chip
    // (8.8 us with eight chunks, 9.9 with four).  A 256-lane collect pass for many rows
    // measured slower (12.5 vs 11.6 us).
    constexpr int kHMax = 4;
    auto per_group = [&](int most, int limit) {
        int g = 1;
        while (g < most && (int64_t)p.rows * ((w.n_chunks + g - 1) / g) > limit) g *= 2;
        return g;
    };
    const bool few = (int64_t)p.rows * w.n_chunks <= kWaveOfGroups;
    const int hs = per_group(kHMax, 2 * kWaveOfGroups);
    const int gsz = per_group((few ? kCTFew : kCTMany) / 64, kWaveOfGroups / 2);
    const unsigned hgrid = (unsigned)(p.rows * ((w.n_chunks + hs - 1) / hs)), cgrid = (unsigned)(p.rows * w.n_chunks);
    const unsigned fgrid = (unsigned)(p.rows * ((w.n_chunks + gsz - 1) / gsz));
    if (few) {
        hipLaunchKernelGGL(k_hist<kCTFew>, dim3(hgrid), dim3(kCTFew), 0, stream, p, w, hs);
        hipLaunchKernelGGL(k_collect<kCTFew>, dim3(cgrid), dim3(kCTFew), 0, stream, p, w);
        hipLaunchKernelGGL(k_finish<kCTFew>, dim3(fgrid), dim3(kCTFew), 0, stream, p, w, gsz);
    } else {
        hipLaunchKernelGGL(k_hist<kCTMany>, dim3(hgrid), dim3(kCTMany), 0, stream, p, w, hs);
        hipLaunchKernelGGL(k_collect<kCTMany>, dim3(cgrid), dim3(kCTMany), 0, stream, p, w);
        hipLaunchKernelGGL(k_finish<kCTMany>, dim3(fgrid), dim3(kCTMany), 0, stream, p, w, gsz);
    }
    return hipGetLastError();
}

}  // namespace fp4idx
