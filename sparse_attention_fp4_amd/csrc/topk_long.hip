// topk_long.hip -- exact top-k over long score rows (more columns than one workgroup
// holds), spread over many workgroups, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Same order and output as topk.hip (larger first, ties to the smaller column, -inf
// and NaN never selected, result in increasing column order, -1 padded).  Scores map
// to order-preserving 32-bit keys; digit 1 is key bits [31:20], digit 2 bits [19:8].
// A row is cut into chunks of 4096 columns.  Workgroups exchange data only across
// kernel boundaries (a device-wide fence inside a kernel costs microseconds on this
// multi-die part):
//   1. hist:    each chunk builds the histogram of digit 1 of its keys in LDS and adds
//               its nonzero bins to the row's histogram (global atomics).
//   2. collect: each chunk reads the row's histogram, finds the bin d1 holding the
//               row's k-th largest key, stores a bitmap of its columns above d1 (all
//               selected) and its keys in d1 (the candidates, with their columns and
//               count), and adds the digit-2 histogram of those candidates to the
//               row's second histogram.
//   3. finish:  one workgroup per row reads the second histogram, the candidate counts,
//               the bitmap and the first slots of every chunk's candidates in one
//               round of loads (a chunk with more candidates sends the workgroup
//               through a slower path that reloads them), finds the digit-2 bin d2 holding
//               the k-th key, selects every candidate above prefix (d1, d2), ranks the
//               few candidates inside it by direct comparison (a digit-pass fallback
//               handles more than 1024 of them), writes the columns in order from
//               popcount scans of the bitmap, and clears its histograms and counter
//               for the next call.
// The workspace must be zero-filled before its first use; every call leaves the
// histograms zero-filled again.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kChunk = 4096;          // columns per chunk workgroup
constexpr int kCT = 512;            // threads of a chunk workgroup: 8 keys per thread
                                    // (its waves run one per SIMD)
constexpr int kPer = kChunk / kCT;    // elements per thread
static_assert(kPer * (kCT / 64) == 64, "the collect scan covers 64 (step, wave) blocks");
constexpr int kBins = 4096;
constexpr int kWords = kChunk / 32;   // bitmap words per chunk
constexpr int kMaxChunks = 128;    // rows of up to 524288 columns
constexpr int kMaxWords = kMaxChunks * kWords;
constexpr int kMaxK = 8192;

struct RowState {
    int d1;         // digit-1 bin of the k-th largest key, or -1 when every valid key is kept
    int kk;         // wanted keys inside bin d1
};

struct LongWs {
    RowState* st;        // [rows]
    uint32_t* hist;      // [rows][kBins]            digit 1 of the keys; zero between calls
    uint32_t* hist2;     // [rows][kBins]            digit 2 of the candidates; zero between calls
    uint32_t* bitmap;    // [rows][n_chunks * kWords] columns above bin d1 (+ selected candidates)
    uint2* cand;         // [rows][n_chunks][kChunk]  candidates (bin d1): (key, column), column order
    int32_t* cnum;       // [rows][n_chunks]          candidates per chunk
    int n_chunks;
    size_t zero_end;     // bytes from the base through hist2: zero when a call starts
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

// Thread t holds elements t + kCT * j of the chunk (index order = j, wave, lane).
__device__ __forceinline__ void load_chunk(const TopkParams& p, int row, int chunk, uint32_t (&key)[kPer]) {
    const int len = row_len(p, row);
    const int c0 = chunk * kChunk;
    const int n = max(0, min(len - c0, kChunk));
    const float* src = p.scores + (int64_t)row * p.row_stride + c0;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int i = threadIdx.x + kCT * j;
        v[j] = i < n ? src[i] : -__builtin_inff();
    }
#pragma unroll
    for (int j = 0; j < kPer; j++) key[j] = to_key(v[j]);
}

// ---------------------------------------------------------------- 1. hist
__global__ __launch_bounds__(kCT) void k_hist(const TopkParams p, LongWs ws) {
    __shared__ uint32_t h[kBins];
    const int row = blockIdx.x / ws.n_chunks, chunk = blockIdx.x - row * ws.n_chunks;
    if (row >= p.rows) return;
    for (int i = threadIdx.x; i < kBins; i += kCT) h[i] = 0u;
    uint32_t key[kPer];
    load_chunk(p, row, chunk, key);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kPer; j++)
        if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
    lds_barrier();
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kCT)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------- 2. collect
struct CollectShared {
    uint32_t h2[kBins];
    int wtot[kCT / 64];
    int pick[4];
    int total;
    uint32_t bits[kWords];
    int cnt[kPer * (kCT / 64)];
    int off[kPer * (kCT / 64)];
};

// The bin of the row's k-th largest key from the row's histogram.  Returns d1 (-1 when
// every valid key is kept) and kk, the keys wanted in d1.
__device__ __forceinline__ void row_threshold_bin(CollectShared& sh, const TopkParams& p, const LongWs& ws,
                                                  int row, int& d1, int& kk) {
    constexpr int per = kBins / kCT;
    int c[per], bin[per];
    const uint32_t* gh = ws.hist + (int64_t)row * kBins;
#pragma unroll
    for (int b = 0; b < per; b++) {  // walked from the top: "before" = larger keys
        bin[b] = kBins - 1 - (threadIdx.x * per + b);
        c[b] = (int)gh[bin[b]];
    }
    pick_bin<kCT, per>(c, bin, p.k, sh.wtot, sh.pick);
    if (sh.pick[2] <= p.k) {
        d1 = -1;
        kk = 0;
    } else {
        d1 = sh.pick[0];
        kk = p.k - sh.pick[1];
    }
}

__global__ __launch_bounds__(kCT) void k_collect(const TopkParams p, LongWs ws) {
    __shared__ CollectShared sh;
    const int row = blockIdx.x / ws.n_chunks, chunk = blockIdx.x - row * ws.n_chunks;
    if (row >= p.rows) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nch = ws.n_chunks;
    uint32_t key[kPer];
    load_chunk(p, row, chunk, key);  // in flight with the histogram loads
    for (int i = threadIdx.x; i < kBins; i += kCT) sh.h2[i] = 0u;
    int d1, kk;
    row_threshold_bin(sh, p, ws, row, d1, kk);  // ends with a barrier
    const int c0 = chunk * kChunk;

    // ---- bitmap of the columns above bin d1; candidates of bin d1 and their digit 2
    bool cand[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const uint32_t kj = key[j];
        const int dig = (int)(kj >> 20);
        const bool above = kj != 0u && (d1 < 0 || dig > d1);
        // a wave covers 64 consecutive columns = two bitmap words
        const unsigned long long ma = __ballot(above);
        const int w0 = (threadIdx.x + kCT * j) >> 5;
        if (lane == 0) sh.bits[w0] = (uint32_t)ma;
        if (lane == 32) sh.bits[w0] = (uint32_t)(ma >> 32);
        cand[j] = d1 >= 0 && kj != 0u && dig == d1;
        const unsigned long long mc = __ballot(cand[j]);
        if (lane == 0) sh.cnt[j * (kCT / 64) + wave] = __popcll(mc);
        if (cand[j]) atomicAdd(&sh.h2[(kj >> 8) & 0xfffu], 1u);
    }
    lds_barrier();
    if (wave == 0) {  // exclusive scan over the kPer * kCT / 64 = 64 (step, wave) blocks
        const int x = sh.cnt[lane];
        const int s = wave_incl_scan(x);
        sh.off[lane] = s - x;
        if (lane == 63) sh.total = s;
    }
    lds_barrier();
    // Global writes come last: a barrier after them would wait for their completion.
    uint2* dst = ws.cand + ((int64_t)row * nch + chunk) * kChunk;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const unsigned long long mc = __ballot(cand[j]);
        if (cand[j]) {
            const int pos = sh.off[j * (kCT / 64) + wave] + lanes_below(mc);
            dst[pos] = make_uint2(key[j], (uint32_t)(c0 + threadIdx.x + kCT * j));
        }
    }
    uint32_t* gbits = ws.bitmap + (int64_t)row * nch * kWords + chunk * kWords;
    for (int i = threadIdx.x; i < kWords; i += kCT) gbits[i] = sh.bits[i];
    if (threadIdx.x == 0) {
        ws.cnum[(int64_t)row * nch + chunk] = sh.total;
        if (chunk == 0) {
            ws.st[row].d1 = d1;
            ws.st[row].kk = kk;
        }
    }
    // the chunk's digit-2 counts join the row's second histogram
    uint32_t* gh2 = ws.hist2 + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kCT) {
        const uint32_t v = sh.h2[i];
        if (v) atomicAdd(&gh2[i], v);
    }
}

// ---------------------------------------------------------------- 3. finish
constexpr int kFT = 1024;    // threads of the finishing workgroup
constexpr int kCR = 8;       // candidates per thread per round
constexpr int kRankMax = 1024;  // candidates at the threshold prefix ranked by comparison

struct FinishShared {
    alignas(16) uint32_t h[kBins];
    uint32_t bits[kMaxWords];  // the row's bitmap
    uint32_t mkey[kRankMax];   // candidates with the threshold prefix (d1, d2)
    int mcol[kRankMax];
    int cnum[kMaxChunks];
    int coff[kMaxChunks + 1];  // candidate prefix over chunks
    int wtot[kFT / 64];
    int pick[4];
    int nm;
};

// Candidate registers: kCR per thread.  In the common case they hold every candidate
// of the row (registers 2j and 2j+1 hold slots 2q % spec and 2q % spec + 1 of chunk
// 2q / spec, q = threadIdx.x + kFT * j);
// otherwise ("flat" mode) they hold candidates [round * kFT * kCR, +kFT * kCR) of the
// row in chunk order, reloaded round by round.
struct CandRegs {
    uint32_t key[kCR];
    int col[kCR];  // -1: no candidate
};

// Candidate i of the row (flat order) lives in chunk c with coff[c] <= i < coff[c+1].
__device__ __forceinline__ int64_t cand_slot(const FinishShared& sh, int row, int nch, int i) {
    int lo = 0, hi = nch;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.coff[mid] <= i) lo = mid;
        else hi = mid;
    }
    return ((int64_t)row * nch + lo) * kChunk + (i - sh.coff[lo]);
}

__device__ __forceinline__ void load_flat(CandRegs& r, const FinishShared& sh, const LongWs& ws, int row,
                                          int nch, int m, int round) {
    uint2 v[kCR];
#pragma unroll
    for (int j = 0; j < kCR; j++) {
        const int i = round * kFT * kCR + threadIdx.x + kFT * j;
        v[j] = i < m ? ws.cand[cand_slot(sh, row, nch, i)] : make_uint2(0u, 0xffffffffu);
    }
#pragma unroll
    for (int j = 0; j < kCR; j++) {
        r.key[j] = v[j].x;
        r.col[j] = (int)v[j].y;
    }
}

// One digit pass over the candidates that pass `keep`: histogram of digit(key, col)
// and the bin holding the kk-th element in the given order.
template <typename Keep, typename Digit>
__device__ __forceinline__ void cand_pass(FinishShared& sh, CandRegs& r, const LongWs& ws, int row, int nch,
                                          int m, int rounds, bool flat, int kk, bool descending, Keep keep,
                                          Digit digit) {
    for (int i = threadIdx.x; i < kBins; i += kFT) sh.h[i] = 0u;
    lds_barrier();
    for (int round = 0; round < rounds; round++) {
        if (flat) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
        for (int j = 0; j < kCR; j++)
            if (r.col[j] >= 0 && keep(r.key[j], r.col[j])) atomicAdd(&sh.h[digit(r.key[j], r.col[j])], 1u);
    }
    lds_barrier();
    constexpr int per = kBins / kFT;
    int c[per], bin[per];
#pragma unroll
    for (int b = 0; b < per; b++) {
        bin[b] = descending ? kBins - 1 - (threadIdx.x * per + b) : threadIdx.x * per + b;
        c[b] = (int)sh.h[bin[b]];
    }
    pick_bin<kFT, per>(c, bin, kk, sh.wtot, sh.pick);
}

__global__ __launch_bounds__(kFT) void k_finish(const TopkParams p, LongWs ws) {
    __shared__ FinishShared sh;
    const int row = blockIdx.x;
    if (row >= p.rows) return;
    const int nch = ws.n_chunks;
    const int k = p.k;
    const int nwords = nch * kWords;
    const uint32_t* rbits = ws.bitmap + (int64_t)row * nch * kWords;
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    uint32_t* gh2 = ws.hist2 + (int64_t)row * kBins;
    constexpr int lspec = 6;            // candidate slots read per chunk up front: 64
    constexpr int spec = 1 << lspec;
    static_assert(kMaxChunks * spec == kFT * kCR && kCR % 2 == 0 && kMaxWords % (4 * kFT) == 0,
                  "up-front loads fill the candidate registers in slot pairs");

    // ---- one round of loads: state, candidate counts, second histogram, bitmap, and the
    // first `spec` candidate slots of every chunk (read before the counts are known;
    // slots past a count are ignored).  This workgroup is alone on its CU, where the
    // number of load instructions, not their latency, sets the pace: every array is read
    // 16 bytes per lane.
    // the digit-1 histogram was last read by the collect pass: clear it for the next
    // call now, so the stores drain while this workgroup works
    static_assert(kBins == 4 * kFT, "one 16-byte store per thread clears a histogram");
    reinterpret_cast<uint4*>(gh)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    const int d1 = ws.st[row].d1;
    int kk = ws.st[row].kk;
    const int my_cnum = threadIdx.x < nch ? ws.cnum[(int64_t)row * nch + threadIdx.x] : 0;
    // second histogram: thread t owns bins 4095-4t .. 4092-4t (one 16-byte load)
    constexpr int per = kBins / kFT;
    uint4* h2v = reinterpret_cast<uint4*>(gh2) + (kFT - 1 - threadIdx.x);
    const uint4 h2 = *h2v;
    int c2[per] = {(int)h2.w, (int)h2.z, (int)h2.y, (int)h2.x}, bin2[per];
#pragma unroll
    for (int b = 0; b < per; b++) bin2[b] = kBins - 1 - (threadIdx.x * per + b);
    // bitmap: words 4q .. 4q+3 for q = threadIdx.x + kFT * j
    constexpr int kXQ = kMaxWords / (4 * kFT);
    const uint4* rbits4 = reinterpret_cast<const uint4*>(rbits);
    uint4 x[kXQ];
#pragma unroll
    for (int j = 0; j < kXQ; j++) {
        const int q = threadIdx.x + kFT * j;
        x[j] = 4 * q < nwords ? rbits4[q] : make_uint4(0u, 0u, 0u, 0u);
    }
    // candidate slot pairs: pair q = threadIdx.x + kFT * j holds slots 2q % spec and
    // 2q % spec + 1 of chunk 2q / spec
    uint4 sv[kCR / 2];
#pragma unroll
    for (int j = 0; j < kCR / 2; j++) {
        const int q = threadIdx.x + kFT * j;
        const int c = (2 * q) >> lspec, slot = (2 * q) & (spec - 1);
        sv[j] = c < nch ? *reinterpret_cast<const uint4*>(ws.cand + ((int64_t)row * nch + c) * kChunk + slot)
                        : make_uint4(0u, 0xffffffffu, 0u, 0xffffffffu);
    }
#pragma unroll
    for (int j = 0; j < kXQ; j++) {
        const int q = threadIdx.x + kFT * j;
        if (4 * q < nwords) reinterpret_cast<uint4*>(sh.bits)[q] = x[j];
    }
    if (threadIdx.x < nch) sh.cnum[threadIdx.x] = my_cnum;
    if (threadIdx.x == 0) sh.nm = 0;
    {
        int before, total;
        block_excl_scan<kFT>(my_cnum, sh.wtot, before, total);  // barriers inside
        if (threadIdx.x < nch) sh.coff[threadIdx.x] = before;
        if (threadIdx.x == 0) sh.coff[nch] = total;
    }
    const bool flat = __syncthreads_or(my_cnum > spec) != 0;  // also publishes coff
    const int m = sh.coff[nch];
    const int rounds = flat ? (m + kFT * kCR - 1) / (kFT * kCR) : 1;
    CandRegs r;
#pragma unroll
    for (int j = 0; j < kCR / 2; j++) {
        const int q = threadIdx.x + kFT * j;
        const int c = (2 * q) >> lspec, slot = (2 * q) & (spec - 1);
        const int cn = c < nch ? sh.cnum[c] : 0;
        r.key[2 * j] = sv[j].x;
        r.col[2 * j] = slot < cn ? (int)sv[j].y : -1;
        r.key[2 * j + 1] = sv[j].z;
        r.col[2 * j + 1] = slot + 1 < cn ? (int)sv[j].w : -1;
    }

    if (d1 >= 0) {
        // ---- digit 2 from the row's second histogram (pick_bin ends with a barrier)
        pick_bin<kFT, per>(c2, bin2, kk, sh.wtot, sh.pick);
        // each thread has its bins' counts in registers: clear them for the next call
        *h2v = make_uint4(0u, 0u, 0u, 0u);
        const uint32_t preA = ((uint32_t)d1 << 12) | (uint32_t)sh.pick[0];
        kk -= sh.pick[1];                      // keys wanted with prefix preA, >= 1
        const int n_pre = sh.pick[3];          // candidates with prefix preA
        // ---- candidates above the prefix are selected; those at it are collected
        for (int round = 0; round < rounds; round++) {
            if (flat) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
            for (int j = 0; j < kCR; j++) {
                const uint32_t pre = r.key[j] >> 8;
                const int col = r.col[j];
                if (col < 0) continue;
                if (pre > preA) {
                    atomicOr(&sh.bits[col >> 5], 1u << (col & 31));
                } else if (pre == preA && n_pre <= kRankMax) {
                    const int at = atomicAdd(&sh.nm, 1);
                    if (at < kRankMax) {   // n_pre bounds it; the test keeps LDS safe
                        sh.mkey[at] = r.key[j];
                        sh.mcol[at] = col;
                    }
                }
            }
        }
        lds_barrier();
        if (n_pre <= kRankMax) {
            // ---- rank each collected candidate by direct comparison
            const int nm = min(sh.nm, kRankMax);
            for (int t = threadIdx.x; t < nm; t += kFT) {
                const uint32_t kt = sh.mkey[t];
                const int ct = sh.mcol[t];
                int rank = 0;
                for (int u = 0; u < nm; u++) {
                    const uint32_t ku = sh.mkey[u];
                    rank += (ku > kt || (ku == kt && sh.mcol[u] < ct)) ? 1 : 0;
                }
                if (rank < kk) atomicOr(&sh.bits[ct >> 5], 1u << (ct & 31));
            }
        } else {
            // ---- many candidates share the prefix: digit passes over them
            cand_pass(sh, r, ws, row, nch, m, rounds, flat, kk, true,
                      [&](uint32_t kx, int) { return (kx >> 8) == preA; },
                      [&](uint32_t kx, int) { return (int)(kx & 0xffu); });
            const uint32_t T = (preA << 8) | (uint32_t)sh.pick[0];
            kk -= sh.pick[1];  // ties at T to keep, >= 1
            const int ties = sh.pick[3];
            int c_cut = 0x7fffffff;
            if (kk < ties) {
                // the kk-th smallest column among the ties at T: bits [30:20], [19:8], [7:0]
                cand_pass(sh, r, ws, row, nch, m, rounds, flat, kk, false, [&](uint32_t kx, int) { return kx == T; },
                          [&](uint32_t, int col) { return (int)(((uint32_t)col >> 20) & 0x7ffu); });
                const uint32_t c1 = (uint32_t)sh.pick[0];
                kk -= sh.pick[1];
                cand_pass(sh, r, ws, row, nch, m, rounds, flat, kk, false,
                          [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 20) == c1; },
                          [&](uint32_t, int col) { return (int)(((uint32_t)col >> 8) & 0xfffu); });
                const uint32_t c2 = (c1 << 12) | (uint32_t)sh.pick[0];
                kk -= sh.pick[1];
                cand_pass(sh, r, ws, row, nch, m, rounds, flat, kk, false,
                          [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 8) == c2; },
                          [&](uint32_t, int col) { return (int)((uint32_t)col & 0xffu); });
                c_cut = (int)((c2 << 8) | (uint32_t)sh.pick[0]);
            }
            for (int round = 0; round < rounds; round++) {
                if (flat) load_flat(r, sh, ws, row, nch, m, round);
#pragma unroll
                for (int j = 0; j < kCR; j++) {
                    const uint32_t kx = r.key[j];
                    const int col = r.col[j];
                    if (col >= 0 && (kx >> 8) == preA && (kx > T || (kx == T && col <= c_cut)))
                        atomicOr(&sh.bits[col >> 5], 1u << (col & 31));
                }
            }
        }
    }
    lds_barrier();

    // ---- columns in order: thread t owns words [t*wpt, (t+1)*wpt) of the bitmap; a
    // block scan of their popcounts gives each thread its output offset
    const float* srow = p.scores + (int64_t)row * p.row_stride;
    int32_t* oidx = p.out_idx + (int64_t)row * k;
    float* oval = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
    const int wpt = (nwords + kFT - 1) / kFT;
    const int wa = threadIdx.x * wpt, wb = min(wa + wpt, nwords);
    int cnt = 0;
    for (int w = wa; w < wb; w++) cnt += __popc(sh.bits[w]);
    int pos, done;
    block_excl_scan<kFT>(cnt, sh.wtot, pos, done);
    for (int w = wa; w < wb && pos < k; w++) {
        uint32_t bits = sh.bits[w];
        while (bits && pos < k) {
            const int col = w * 32 + __ffs((int)bits) - 1;
            oidx[pos] = col;
            if (oval) oval[pos] = srow[col];
            pos++;
            bits &= bits - 1u;
        }
    }
    for (int i = min(done, k) + threadIdx.x; i < k; i += kFT) {
        oidx[i] = -1;
        if (oval) oval[i] = -__builtin_inff();
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LongWs carve(void* base, int rows, int cols, size_t* bytes) {
    LongWs w{};
    w.n_chunks = (cols + kChunk - 1) / kChunk;
    const size_t rc = (size_t)rows * w.n_chunks;
    unsigned char* b = reinterpret_cast<unsigned char*>(base);
    size_t o = 0;
    w.st = reinterpret_cast<RowState*>(b + o);
    o = align256(o + (size_t)rows * sizeof(RowState));
    w.hist = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + (size_t)rows * kBins * 4);
    w.hist2 = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + (size_t)rows * kBins * 4);
    w.zero_end = o;
    w.bitmap = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + rc * kWords * 4);
    w.cand = reinterpret_cast<uint2*>(b + o);
    o = align256(o + rc * kChunk * sizeof(uint2));
    w.cnum = reinterpret_cast<int32_t*>(b + o);
    o = align256(o + rc * 4);
    if (bytes) *bytes = o;
    return w;
}

}  // namespace

// Rows longer than one workgroup holds go here; so do rows of more than 8192 columns
// when there are few of them: spread over chunk workgroups they finish sooner than with
// one workgroup per row (4 rows of 16384 columns: 14.5 against 16.5 us), while many
// rows keep the chip busy one workgroup each.
bool topk_long_rows(int rows, int cols) { return cols > 32768 || (cols > 8192 && rows <= 64); }

// Leading workspace bytes that must be zero when a call starts: the row states and the
// two histograms come first in the layout (a caller that cannot keep the workspace
// between calls clears just these).
size_t topk_long_zero_bytes(int rows, int cols) { return carve(nullptr, rows, cols, nullptr).zero_end; }

size_t topk_long_workspace_bytes(int rows, int cols, int k) {
    (void)k;
    size_t bytes = 0;
    carve(nullptr, rows, cols, &bytes);
    return bytes;
}

hipError_t launch_topk_long(const TopkParams& p, void* workspace, hipStream_t stream) {
    LongWs w = carve(workspace, p.rows, p.cols, nullptr);
    if (w.n_chunks > kMaxChunks) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(p.rows * w.n_chunks);
    hipLaunchKernelGGL(k_hist, dim3(grid), dim3(kCT), 0, stream, p, w);
    hipLaunchKernelGGL(k_collect, dim3(grid), dim3(kCT), 0, stream, p, w);
    hipLaunchKernelGGL(k_finish, dim3(p.rows), dim3(kFT), 0, stream, p, w);
    return hipGetLastError();
}

}  // namespace fp4idx
