// topk_long.hip -- exact top-k over long score rows (more columns than one workgroup
// holds), spread over many workgroups, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Same order and output as topk.hip (larger first, ties to the smaller column, -inf
// and NaN never selected, result in increasing column order, -1 padded).  A row is cut
// into chunks of 4096 columns.  Workgroups exchange data only across kernel
// boundaries (a device-wide fence inside a kernel costs microseconds on this
// multi-die part):
//   1. hist:    each chunk builds the histogram of the top 12 key bits of its elements
//               in LDS and adds its nonzero bins to the row's histogram (global
//               atomics that nothing waits for).
//   2. collect: each chunk reads the row's histogram, finds the bin d1 that holds the
//               row's k-th largest key, and stores a bitmap of its columns above d1
//               (all selected) and, in column order, the keys and columns in d1 (the
//               candidates).
//   3. finish:  one workgroup per row narrows the candidates to the exact threshold key
//               T (two more digit passes over candidates kept in registers), finds the
//               column cut among ties at T, ORs the selected candidates into an LDS copy
//               of the row's bitmap, writes the columns in order from a popcount scan,
//               gathers their scores, and clears the row's histogram for the next call.
// Every phase issues its global loads together: a round trip costs about a
// microsecond here.  The workspace must be zero-filled before its first use; every
// call leaves the histograms zero-filled again.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kChunk = 4096;          // columns per chunk workgroup
constexpr int kCT = 256;              // threads of a workgroup
constexpr int kPer = kChunk / kCT;    // elements per thread
constexpr int kBins = 4096;
constexpr int kWords = kChunk / 32;   // bitmap words per chunk
constexpr int kMaxChunks = 128;    // rows of up to 524288 columns
constexpr int kMaxWords = kMaxChunks * kWords;
constexpr int kMaxK = 8192;

struct RowState {
    int d1;         // bin of the k-th largest key, or -1 when every valid key is kept
    int kk;         // wanted keys inside bin d1
};

struct LongWs {
    RowState* st;        // [rows]
    uint32_t* hist;      // [rows][kBins]            zero between calls
    uint32_t* bitmap;    // [rows][n_chunks * kWords] columns above bin d1 (+ selected candidates)
    uint32_t* ckey;      // [rows][n_chunks][kChunk] candidates (bin d1): keys, in column order
    int32_t* ccol;       // [rows][n_chunks][kChunk] candidates: columns
    int32_t* cnum;       // [rows][n_chunks]         candidates per chunk
    int n_chunks;
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
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; j++)
        if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
    __syncthreads();
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kCT)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------- 2. collect
struct CollectShared {
    int wtot[kCT / 64];
    int pick[3];
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
    int d1, kk;
    row_threshold_bin(sh, p, ws, row, d1, kk);
    if (chunk == 0 && threadIdx.x == 0) {
        ws.st[row].d1 = d1;
        ws.st[row].kk = kk;
    }
    const int c0 = chunk * kChunk;

    // ---- bitmap of the columns above bin d1; candidates of bin d1 in column order
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
    }
    __syncthreads();
    uint32_t* gbits = ws.bitmap + (int64_t)row * nch * kWords + chunk * kWords;
    for (int i = threadIdx.x; i < kWords; i += kCT) gbits[i] = sh.bits[i];
    if (wave == 0) {  // exclusive scan over the kPer * 4 = 64 (step, wave) blocks
        const int x = sh.cnt[lane];
        int s = x;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(s, d);
            if (lane >= d) s += y;
        }
        sh.off[lane] = s - x;
        if (lane == 63) ws.cnum[(int64_t)row * nch + chunk] = s;
    }
    __syncthreads();
    const int64_t base = ((int64_t)row * nch + chunk) * kChunk;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const unsigned long long mc = __ballot(cand[j]);
        if (cand[j]) {
            const int pos = sh.off[j * (kCT / 64) + wave] + lanes_below(mc);
            ws.ckey[base + pos] = key[j];
            ws.ccol[base + pos] = c0 + threadIdx.x + kCT * j;
        }
    }
}

// ---------------------------------------------------------------- 3. finish
constexpr int kFT = 1024;  // threads of the finishing workgroup

struct FinishShared {
    uint32_t h[kBins];
    uint32_t bits[kMaxWords];  // the row's bitmap
    int sel[kMaxK];            // selected columns in order
    int coff[kMaxChunks + 1];  // candidate prefix over chunks
    int wtot[kFT / 64];
    int pick[3];
};

// Candidate i of the row lives in chunk c with coff[c] <= i < coff[c+1].
__device__ __forceinline__ int64_t cand_slot(const FinishShared& sh, int row, int nch, int i) {
    int lo = 0, hi = nch;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.coff[mid] <= i) lo = mid;
        else hi = mid;
    }
    return ((int64_t)row * nch + lo) * kChunk + (i - sh.coff[lo]);
}

// The candidates of the row, kCR per thread per round (candidate i = round * kFT * kCR
// + threadIdx.x + kFT * j); a row with at most kFT * kCR candidates keeps them in
// registers for all passes, a larger one reloads them round by round.
constexpr int kCR = 8;

struct CandRegs {
    uint32_t key[kCR];
    int col[kCR];  // -1: no candidate
};

__device__ __forceinline__ void load_round(CandRegs& r, const FinishShared& sh, const LongWs& ws, int row,
                                           int nch, int m, int round) {
#pragma unroll
    for (int j = 0; j < kCR; j++) {
        const int i = round * kFT * kCR + threadIdx.x + kFT * j;
        r.key[j] = 0u;
        r.col[j] = -1;
        if (i < m) {
            const int64_t at = cand_slot(sh, row, nch, i);
            r.key[j] = ws.ckey[at];
            r.col[j] = ws.ccol[at];
        }
    }
}

// One digit pass over the candidates that pass `keep`: histogram of digit(key, col)
// and the bin holding the kk-th element in the given order.
template <typename Keep, typename Digit>
__device__ __forceinline__ void cand_pass(FinishShared& sh, CandRegs& r, const LongWs& ws, int row, int nch,
                                          int m, int rounds, int kk, bool descending, Keep keep, Digit digit) {
    for (int i = threadIdx.x; i < kBins; i += kFT) sh.h[i] = 0u;
    __syncthreads();
    for (int round = 0; round < rounds; round++) {
        if (rounds > 1) load_round(r, sh, ws, row, nch, m, round);
        const int left = m - round * kFT * kCR;  // candidates of this round
#pragma unroll
        for (int j = 0; j < kCR; j++) {
            // slot j holds candidates only below `left` (a uniform test)
            if (kFT * j < left && r.col[j] >= 0 && keep(r.key[j], r.col[j]))
                atomicAdd(&sh.h[digit(r.key[j], r.col[j])], 1u);
        }
    }
    __syncthreads();
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
    // ---- the row's bitmap into LDS (loads in flight together)
    for (int w = threadIdx.x; w < nwords; w += kFT * 16) {
        uint32_t x[16];
#pragma unroll
        for (int j = 0; j < 16; j++) x[j] = w + kFT * j < nwords ? rbits[w + kFT * j] : 0u;
#pragma unroll
        for (int j = 0; j < 16; j++)
            if (w + kFT * j < nwords) sh.bits[w + kFT * j] = x[j];
    }
    const int d1 = ws.st[row].d1;
    int kk = ws.st[row].kk;
    {
        const int c = threadIdx.x;  // nch <= kMaxChunks <= kFT
        const int v = c < nch ? ws.cnum[(int64_t)row * nch + c] : 0;
        int before, total;
        block_excl_scan<kFT>(v, sh.wtot, before, total);
        if (c < nch) sh.coff[c] = before;
        if (threadIdx.x == 0) sh.coff[nch] = total;
    }
    __syncthreads();
    const int m = sh.coff[nch];
    if (d1 >= 0) {
        const int rounds = (m + kFT * kCR - 1) / (kFT * kCR);
        CandRegs r;
        load_round(r, sh, ws, row, nch, m, 0);
        cand_pass(sh, r, ws, row, nch, m, rounds, kk, true, [&](uint32_t, int) { return true; },
                  [&](uint32_t kx, int) { return (int)((kx >> 8) & 0xfffu); });
        const uint32_t preA = ((uint32_t)d1 << 12) | (uint32_t)sh.pick[0];
        kk -= sh.pick[1];
        cand_pass(sh, r, ws, row, nch, m, rounds, kk, true, [&](uint32_t kx, int) { return (kx >> 8) == preA; },
                  [&](uint32_t kx, int) { return (int)(kx & 0xffu); });
        const uint32_t T = (preA << 8) | (uint32_t)sh.pick[0];
        kk -= sh.pick[1];  // ties at T to keep, >= 1
        const int ties = (int)sh.h[sh.pick[0]];
        __syncthreads();
        int c_cut = 0x7fffffff;
        if (kk < ties) {
            // the kk-th smallest column among the ties at T: bits [30:20], [19:8], [7:0]
            cand_pass(sh, r, ws, row, nch, m, rounds, kk, false, [&](uint32_t kx, int) { return kx == T; },
                      [&](uint32_t, int col) { return (int)(((uint32_t)col >> 20) & 0x7ffu); });
            const uint32_t c1 = (uint32_t)sh.pick[0];
            kk -= sh.pick[1];
            cand_pass(sh, r, ws, row, nch, m, rounds, kk, false,
                      [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 20) == c1; },
                      [&](uint32_t, int col) { return (int)(((uint32_t)col >> 8) & 0xfffu); });
            const uint32_t c2 = (c1 << 12) | (uint32_t)sh.pick[0];
            kk -= sh.pick[1];
            cand_pass(sh, r, ws, row, nch, m, rounds, kk, false,
                      [&](uint32_t kx, int col) { return kx == T && ((uint32_t)col >> 8) == c2; },
                      [&](uint32_t, int col) { return (int)((uint32_t)col & 0xffu); });
            c_cut = (int)((c2 << 8) | (uint32_t)sh.pick[0]);
        }
        // selected candidates join the bitmap
        for (int round = 0; round < rounds; round++) {
            if (rounds > 1) load_round(r, sh, ws, row, nch, m, round);
#pragma unroll
            for (int j = 0; j < kCR; j++) {
                const uint32_t kx = r.key[j];
                const int col = r.col[j];
                if (col >= 0 && (kx > T || (kx == T && col <= c_cut))) atomicOr(&sh.bits[col >> 5], 1u << (col & 31));
            }
        }
    }
    __syncthreads();

    // ---- columns in order: thread t scans words [t*wpt, (t+1)*wpt) of the LDS bitmap
    const int wpt = (nwords + kFT - 1) / kFT;
    const int w0 = threadIdx.x * wpt, w1 = min(w0 + wpt, nwords);
    int s = 0;
    for (int w = w0; w < w1; w++) s += __popc(sh.bits[w]);
    int pos, total;
    block_excl_scan<kFT>(s, sh.wtot, pos, total);
    for (int w = w0; w < w1 && pos < k; w++) {
        uint32_t bits = sh.bits[w];
        while (bits && pos < k) {
            sh.sel[pos++] = w * 32 + __ffs((int)bits) - 1;
            bits &= bits - 1u;
        }
    }
    __syncthreads();
    // ---- output, coalesced; the scores come in with all loads in flight
    const int n_out = min(total, k);
    const float* srow = p.scores + (int64_t)row * p.row_stride;
    for (int base = 0; base < k; base += kFT * 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int i = base + threadIdx.x + kFT * j;
            v[j] = (p.out_vals && i < n_out) ? srow[sh.sel[i]] : -__builtin_inff();
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int i = base + threadIdx.x + kFT * j;
            if (i < k) {
                p.out_idx[(int64_t)row * k + i] = i < n_out ? sh.sel[i] : -1;
                if (p.out_vals) p.out_vals[(int64_t)row * k + i] = v[j];
            }
        }
    }
    // ---- leave the row's histogram zero-filled for the next call
    uint32_t* gh = ws.hist + (int64_t)row * kBins;
    for (int i = threadIdx.x; i < kBins; i += kFT) gh[i] = 0u;
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
    w.bitmap = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + rc * kWords * 4);
    w.ckey = reinterpret_cast<uint32_t*>(b + o);
    o = align256(o + rc * kChunk * 4);
    w.ccol = reinterpret_cast<int32_t*>(b + o);
    o = align256(o + rc * kChunk * 4);
    w.cnum = reinterpret_cast<int32_t*>(b + o);
    o = align256(o + rc * 4);
    if (bytes) *bytes = o;
    return w;
}

}  // namespace

bool topk_long_rows(int cols) { return cols > 32768; }

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
