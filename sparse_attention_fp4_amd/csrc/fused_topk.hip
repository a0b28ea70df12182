// fused_topk.hip -- weighted-ReLU scores and their top-k without writing the logits,
// gfx950.
//
// ("Lightning Indexer FP4 dequant decodes E2M1 wrong" issue, "Fix (production target)":
// scores accumulated on the matrix cores, ReLU and head weights in the epilogue, top-k
// selected without a serial heap -- the scorer and the selection as one unit.)
//
// The result equals fp4idx_topk over the logits fp4idx_logits_paged writes (same
// scores, same rule: the k largest finite scores of the visible columns, ties to the
// smaller column, increasing column order, -1 padding), but the T x out_cols score
// matrix never goes to memory.  Steps, all on the device:
//   1. sampled table: every 16th logical page of each request (the row lengths mapped
//      onto the sampled columns);
//   2. the scorer over the sampled pages (1/16 of the work) writes their scores;
//   3. per row, lo = the m-th largest sampled score, m = 2 ceil(k / 16) (about 2k
//      scores of the full row reach it), or -inf when fewer than m are finite;
//   4. the scorer over every page keeps only the scores >= lo, as (value, column)
//      entries packed at the start of each wave's own column range (no atomics; only
//      the kept entries are written);
//   5. per row, the exact top-k of the kept entries.  Every score >= lo was kept, so
//      when at least k were kept the top k are among them.  A row with fewer (only
//      possible when lo > -inf) is flagged;
//   6. the scorer runs again for the row blocks holding a flagged row, keeping every
//      score of those rows, and the selection is redone for them (both launches find
//      nothing to do when no row is flagged).
// That pipeline pays off with many rows (prefill).  With fewer than 512 rows the
// logits do go to the workspace, and the plain top-k selects from them.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kSampleStride = 16;   // one logical page in 16 is scored first
constexpr int kSelThreads = 256;
constexpr int kMaxChunks = 32767;   // column chunks per row (their prefix lives in LDS)
constexpr int kSortCap = 2048;      // largest k

__device__ __forceinline__ uint32_t order_key(uint32_t u) {
    if (u == 0x80000000u) u = 0u;   // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_value_bits(uint32_t key) {
    return (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
}

struct SampleParams {
    const int32_t* bt;  // [B][bt_rs]
    int64_t bt_rs;
    int B, W, Ws;
    const int32_t* lens;
    int T, out_cols, page;
    int32_t* bt_s;      // [B][Ws]
    int32_t* lens_s;    // [T]
};

// Sampled block table (logical page 16j of each request becomes sampled page j) and
// the row lengths on the sampled columns: column r of sampled page j is column
// 16 j page + r of the row, visible iff below min(len, out_cols); the visible sampled
// columns are again a prefix.
__global__ __launch_bounds__(256) void k_sample_table(const SampleParams p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < (int64_t)p.B * p.Ws) {
        const int b = (int)(i / p.Ws), j = (int)(i - (int64_t)b * p.Ws);
        const int lp = j * kSampleStride;
        p.bt_s[i] = lp < p.W ? p.bt[(int64_t)b * p.bt_rs + lp] : -1;
    }
    if (i < p.T) {
        const int L = max(0, min(p.lens[i], p.out_cols));
        const int span = kSampleStride * p.page;
        p.lens_s[i] = p.page * (L / span) + min(p.page, L % span);
    }
}

// ---- wave-level reductions and scans (one wave handles one row; no workgroup barriers)
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}
__device__ __forceinline__ void wave_minmax(uint32_t& lo, uint32_t& hi) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, d));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, d));
    }
}

constexpr int kBins = 1024;  // histogram bins of one narrowing step


// One narrowing step of a wave over the keys in [klo, khi] (visit(fn) calls fn(key) for
// each key of the lane): bin (key - klo) >> sh into at most 1024 bins of the wave's LDS
// histogram and find the bin holding the want-th largest key (want counted from the top
// of the range, 1 <= want <= the keys in the range); `above` receives the number of keys
// in higher bins.  Offsets from the range's bottom spread close values over many bins,
// so few lanes add to one bin at a time.
template <class Visit>
__device__ __forceinline__ void wave_narrow(Visit visit, uint32_t klo, uint32_t khi, int want,
                                            int* hist, int& bin, int& above, int& sh) {
    const int lane = threadIdx.x & 63;
    const uint32_t span = khi - klo;
    sh = span >= (uint32_t)kBins ? (32 - __builtin_clz(span)) - 10 : 0;
#pragma unroll
    for (int i = 0; i < kBins / 64; i++) hist[64 * i + lane] = 0;  // consecutive lanes, consecutive banks
    __builtin_amdgcn_wave_barrier();
    const int shv = sh;
    visit([&](uint32_t key) {
        if (key >= klo && key <= khi) atomicAdd(&hist[(key - klo) >> shv], 1);
    });
    __builtin_amdgcn_wave_barrier();
    // lane l holds bins 1023-16l .. 1008-16l, in descending order, read 16 bytes at a
    // time (one word per read would put the lanes' bins, 16 words apart, in few banks)
    constexpr int kPerLane = kBins / 64;
    int c[kPerLane], s = 0;
    const v4i* hv = reinterpret_cast<const v4i*>(hist + kBins - kPerLane * (lane + 1));
#pragma unroll
    for (int q = 0; q < kPerLane / 4; q++) {
        const v4i v = hv[q];
#pragma unroll
        for (int e = 0; e < 4; e++) c[kPerLane - 1 - (4 * q + e)] = v[e];
    }
#pragma unroll
    for (int i = 0; i < kPerLane; i++) s += c[i];
    const int incl = wave_incl_scan(s);
    const int excl = incl - s;
    const unsigned long long hit = __ballot(excl < want && want <= incl);
    const int src = __ffsll((long long)hit) - 1;
    int b = 0, ab = 0, run = excl;
    bool found = false;
#pragma unroll
    for (int i = 0; i < kPerLane; i++) {
        if (!found && run + c[i] >= want) {
            b = kBins - 1 - kPerLane * lane - i;
            ab = run;
            found = true;
        }
        run += c[i];
    }
    bin = __shfl(b, src);
    above = __shfl(ab, src);
    __builtin_amdgcn_wave_barrier();
}

// The want-th largest key (1 <= want <= the keys visited) of a wave: narrowing steps
// from [kmin, kmax], each 1024 times narrower.  *above receives the number of keys
// above the result.
template <class Visit>
__device__ __forceinline__ uint32_t wave_nth_largest(Visit visit, uint32_t kmin, uint32_t kmax,
                                                     int want, int* hist, int* above_out) {
    int above = 0;
    while (kmin < kmax) {  // wave-uniform
        int bin, ab, sh;
        wave_narrow(visit, kmin, kmax, want - above, hist, bin, ab, sh);
        above += ab;
        const uint32_t nlo = kmin + ((uint32_t)bin << sh);
        kmax = min(kmax, nlo + ((1u << sh) - 1u));
        kmin = nlo;
    }
    *above_out = above;
    return kmin;
}

__device__ __forceinline__ int block_sum(int v, int* red) {
    v = wave_sum(v);
    __syncthreads();  // the previous use of red is over
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}
// exclusive prefix of v over the workgroup's lanes in order; *total receives the sum
__device__ __forceinline__ int block_excl_scan(int v, int* red, int* total) {
    const int incl = wave_incl_scan(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    int base = 0;
    for (int i = 0; i < w; i++) base += red[i];
    *total = red[0] + red[1] + red[2] + red[3];
    return base + incl - v;
}

__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* red8) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, d));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, d));
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = lo, red8[4 + (threadIdx.x >> 6)] = hi;
    __syncthreads();
    lo = min(min(red8[0], red8[1]), min(red8[2], red8[3]));
    hi = max(max(red8[4], red8[5]), max(red8[6], red8[7]));
}


struct NarrowLds {
    alignas(16) int hist[kBins];  // read 16 bytes at a time
    int red[4];
    uint32_t red8[8];
    int misc[3];
};

// One narrowing step over the keys in [klo, khi] (visit(fn) calls fn(key) for each key
// of the lane): bin (key - klo) >> sh into at most 1024 bins and find the bin holding
// the want-th largest key (want counted from the top of the range, 1 <= want <= the
// number of keys in the range); `above` receives the number of keys in higher bins,
// `inbin` the number in the bin.
// Offsets from the range's bottom spread close values over many bins, so few lanes
// add to one bin at a time.
template <class Visit>
__device__ __forceinline__ void narrow(Visit visit, uint32_t klo, uint32_t khi, int want,
                                       NarrowLds& L, int& bin, int& above, int& sh, int& inbin) {
    const uint32_t span = khi - klo;
    sh = span >= (uint32_t)kBins ? (32 - __clz((int)span)) - 10 : 0;
    if (span >= 0x80000000u) sh = 22;
    for (int i = threadIdx.x; i < kBins; i += 256) L.hist[i] = 0;
    __syncthreads();
    const int shv = sh;
    visit([&](uint32_t key) {
        if (key >= klo && key <= khi) atomicAdd(&L.hist[(key - klo) >> shv], 1);
    });
    __syncthreads();
    // lane t holds bins 1023-4t .. 1020-4t, in descending order (one 16-byte read)
    int c[4], s = 0;
    {
        const v4i v = *reinterpret_cast<const v4i*>(L.hist + kBins - 4 * ((int)threadIdx.x + 1));
#pragma unroll
        for (int i = 0; i < 4; i++) {
            c[i] = v[3 - i];
            s += c[i];
        }
    }
    int tot;
    const int excl = block_excl_scan(s, L.red, &tot);
    if (excl < want && want <= excl + s) {
        int run = excl;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (run + c[i] >= want) {
                L.misc[0] = kBins - 1 - 4 * (int)threadIdx.x - i;
                L.misc[1] = run;
                L.misc[2] = c[i];
                break;
            }
            run += c[i];
        }
    }
    __syncthreads();
    bin = L.misc[0];
    above = L.misc[1];
    inbin = L.misc[2];
    __syncthreads();
}

constexpr int kThrPer = 48;  // sampled scores per lane held in registers (3072 per row)

struct ThresholdParams {
    const float* slog;   // [T][cols_s]
    const int32_t* lens_s;
    int T, cols_s, m;
    float* lo;           // [T]
};

// lo of each row, one wave per row: the row's sampled scores (at most 3072; a longer
// sample is thinned to every stride-th score, with m divided by the stride) in
// registers; lo = their m-th largest, or -inf when fewer than m are finite.
__global__ __launch_bounds__(256) void k_threshold(const ThresholdParams p) {
    __shared__ __align__(16) int hist_all[4][kBins];  // read 16 bytes at a time
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= p.T) return;  // whole wave; nothing below waits for other waves
    int* hist = hist_all[wave];
    const float* row = p.slog + (int64_t)t * p.cols_s;
    const int S = max(0, min(p.lens_s[t], p.cols_s));
    constexpr int per_wave = 64 * kThrPer;
    const int stride = S > per_wave ? (S + per_wave - 1) / per_wave : 1;
    const int n = (S + stride - 1) / stride;
    const int m = (p.m + stride - 1) / stride;
    uint32_t key[kThrPer];
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    int finite = 0;
#pragma unroll
    for (int i = 0; i < kThrPer; i++) {
        const int j = lane + 64 * i;
        const float v = j < n ? row[(int64_t)j * stride] : -__builtin_inff();
        const bool ok = v > -__builtin_inff();  // -inf and NaN are never chosen
        key[i] = ok ? order_key(__float_as_uint(v)) : 0u;
        finite += ok ? 1 : 0;
        kmin = ok ? min(kmin, key[i]) : kmin;
        kmax = ok ? max(kmax, key[i]) : kmax;
    }
    if (wave_sum(finite) < m) {
        if (lane == 0) p.lo[t] = -__builtin_inff();
        return;
    }
    wave_minmax(kmin, kmax);
    int above;
    const uint32_t kth = wave_nth_largest([&](auto&& fn) {
#pragma unroll
        for (int i = 0; i < kThrPer; i++)
            if (key[i] != 0u) fn(key[i]);
    }, kmin, kmax, m, hist, &above);
    if (lane == 0) p.lo[t] = __uint_as_float(key_value_bits(kth));
}

struct SelectParams {
    const uint64_t* cand;   // [T][cand_rs]
    int64_t cand_rs;
    const int32_t* counts;  // [T][counts_rs]
    int counts_rs, nchunks, chunk_w;
    const float* lo;
    int32_t* flags;
    int second;             // 0: first selection (writes flags), 1: flagged rows only
    int T, k;
    int32_t* out_idx;       // [T][k]
    float* out_vals;        // [T][k] or null
};

constexpr int kSelPer = 24;  // kept entries per lane held in registers (6144 per row)

// Exact top-k of one row's kept entries: one 256-lane workgroup per row.  The entries
// of the row, in chunk order and in column order inside a chunk, are in increasing
// column order; lane l takes a contiguous range of them.  The k-th largest key comes
// from a bit-by-bit count; the ties at it are taken in column order and every chosen
// entry's output position is its rank in that order (two prefix scans, no sorting).
__global__ __launch_bounds__(kSelThreads) void k_fused_select(const SelectParams p) {
    extern __shared__ __align__(16) int pre[];  // [nchunks + 1] prefix of the chunk counts
    __shared__ NarrowLds L;
    int* const red = L.red;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    if (p.second && p.flags[t] == 0) return;  // uniform

    // ---- prefix of the chunk counts (lane l takes consecutive chunks)
    const int nch = p.nchunks;
    const int32_t* cnt = p.counts + (int64_t)t * p.counts_rs;
    const int cper = (nch + kSelThreads - 1) / kSelThreads;
    int sum = 0;
    for (int i = 0; i < cper; i++) {
        const int c = tid * cper + i;
        sum += c < nch ? cnt[c] : 0;
    }
    int N;
    int run = block_excl_scan(sum, red, &N);
    for (int i = 0; i < cper; i++) {
        const int c = tid * cper + i;
        if (c < nch) {
            pre[c] = run;
            run += cnt[c];
        }
    }
    if (tid == 0) pre[nch] = N;
    const float lo_t = p.second ? -__builtin_inff() : p.lo[t];
    if (!p.second) {
        const bool flag = lo_t > -__builtin_inff() && N < p.k;
        if (tid == 0) p.flags[t] = flag ? 1 : 0;
        if (flag) return;  // uniform
    }
    __syncthreads();

    const uint64_t* crow = p.cand + (int64_t)t * p.cand_rs;
    auto fetch = [&](int i) -> uint64_t {  // entry i of the row (its chunk by binary search)
        int a = 0, b = nch;                // pre[a] <= i < pre[b]
        while (b - a > 1) {
            const int mid = (a + b) >> 1;
            if (pre[mid] <= i) a = mid;
            else b = mid;
        }
        return crow[(int64_t)a * p.chunk_w + (i - pre[a])];
    };
    auto key_of = [](uint64_t e) { return order_key((uint32_t)e); };
    const int E = (N + kSelThreads - 1) / kSelThreads;  // entries per lane
    const int i0 = tid * E, i1 = min(N, i0 + E);
    const bool held = E <= kSelPer;                      // entries in registers
    const int mine = max(0, i1 - i0);
    uint64_t ent[kSelPer];
    if (held) {
        // the chunk of the lane's first entry by binary search, then forward: entries are
        // consecutive, so each next one is in the same chunk or a later one
        int a = 0;
        if (mine > 0) {
            int b = nch;
            while (b - a > 1) {
                const int mid = (a + b) >> 1;
                if (pre[mid] <= i0) a = mid;
                else b = mid;
            }
        }
        int64_t off[kSelPer];
#pragma unroll
        for (int j = 0; j < kSelPer; j++) {
            const int i = min(i0 + j, max(i1 - 1, i0));
            while (a + 1 < nch && pre[a + 1] <= i) a++;
            off[j] = (int64_t)a * p.chunk_w + (i - pre[a]);
        }
#pragma unroll
        for (int j = 0; j < kSelPer; j++) ent[j] = j < mine ? crow[off[j]] : 0ull;
    }
    // visit this lane's entries in order (registers: a fully unrolled loop, so the array
    // stays in registers)
    auto visit = [&](auto&& fn) {
        if (held) {
#pragma unroll
            for (int j = 0; j < kSelPer; j++)
                if (j < mine) fn(ent[j]);
        } else {
            for (int j = 0; j < mine; j++) fn(fetch(i0 + j));
        }
    };

    // ---- the k-th largest key and how many of its ties are taken
    const bool all = N <= p.k;
    uint32_t kth = 0;
    int need = 0;
    if (!all) {
        // narrow [smallest, largest key] down to the k-th key; `above` counts the keys
        // above the current range
        uint32_t klo = 0xffffffffu, khi = 0u;
        visit([&](uint64_t e) {
            klo = min(klo, key_of(e));
            khi = max(khi, key_of(e));
        });
        block_minmax(klo, khi, L.red8);
        int above = 0;
        while (klo < khi) {  // uniform; each step shrinks the range 1024-fold
            int bin, ab, sh, inb;
            narrow([&](auto&& fn) { visit([&](uint64_t e) { fn(key_of(e)); }); }, klo, khi,
                   p.k - above, L, bin, ab, sh, inb);
            above += ab;
            const uint32_t nlo = klo + ((uint32_t)bin << sh);
            const uint32_t width = sh >= 32 ? 0xffffffffu : ((1u << sh) - 1u);
            khi = min(khi, nlo + width);
            klo = nlo;
            // every key of the bin is taken: kth = the bin's bottom (need covers any ties
            // at it), no further narrowing
            if (inb == p.k - above) break;
        }
        kth = klo;
        need = p.k - above;  // keys above kth: every key above a range was counted
    }
    // ---- ties in column order, then every chosen entry's output position
    int32_t* oi = p.out_idx + (int64_t)t * p.k;
    float* ov = p.out_vals ? p.out_vals + (int64_t)t * p.k : nullptr;
    int m;
    if (held) {
        // branch-free: flags by arithmetic, stores through descriptors (an entry that is
        // not chosen gets an offset past the row)
        int ties = 0;
#pragma unroll
        for (int j = 0; j < kSelPer; j++) ties += (!all && j < mine && key_of(ent[j]) == kth) ? 1 : 0;
        int tot;
        const int tie0 = block_excl_scan(ties, red, &tot);
        bool ch[kSelPer];
        int take = 0, tr = tie0;
#pragma unroll
        for (int j = 0; j < kSelPer; j++) {
            const uint32_t key = key_of(ent[j]);
            const bool tie = !all && key == kth;
            ch[j] = j < mine && (all || key > kth || (tie && tr < need));
            tr += (j < mine && tie) ? 1 : 0;
            take += ch[j] ? 1 : 0;
        }
        int pos = block_excl_scan(take, red, &m);
        const uint32_t row_bytes = (uint32_t)p.k * 4u;
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(oi, row_bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(ov ? (const void*)ov : (const void*)oi, ov ? row_bytes : 0u);
#pragma unroll
        for (int j = 0; j < kSelPer; j++) {
            const uint32_t o = ch[j] ? (uint32_t)pos * 4u : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(ent[j] >> 32), ri, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)ent[j], rv, o, 0, 0);
            pos += ch[j] ? 1 : 0;
        }
    } else {
        int ties = 0;
        if (!all) visit([&](uint64_t e) { ties += key_of(e) == kth ? 1 : 0; });
        int tot;
        const int tie0 = block_excl_scan(ties, red, &tot);
        auto chosen = [&](uint64_t e, int& tie_rank) {
            if (all) return true;
            const uint32_t key = key_of(e);
            if (key > kth) return true;
            if (key != kth) return false;
            return tie_rank++ < need;
        };
        int take = 0;
        {
            int tr = tie0;
            visit([&](uint64_t e) { take += chosen(e, tr) ? 1 : 0; });
        }
        int pos = block_excl_scan(take, red, &m);
        int tr = tie0;
        visit([&](uint64_t e) {
            if (chosen(e, tr)) {
                oi[pos] = (int32_t)(e >> 32);
                if (ov) ov[pos] = __uint_as_float((uint32_t)e);
                pos++;
            }
        });
    }
    for (int i = m + tid; i < p.k; i += kSelThreads) {
        oi[i] = -1;
        if (ov) ov[i] = -__builtin_inff();
    }
}

__global__ __launch_bounds__(256) void k_fill_empty(int64_t n, int32_t* idx, float* vals) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    idx[i] = -1;
    if (vals) vals[i] = -__builtin_inff();
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__global__ __launch_bounds__(256) void k_zero_words(int64_t n, uint32_t* w) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) w[i] = 0u;
}

// Fewer rows than this: the scorer writes the logits into the workspace and the plain
// top-k selects from them.  The sampled-threshold path pays off when many rows share
// the chip (prefill); with few rows its one-workgroup-per-row selection over each
// row's kept scores is the slow part (4 rows of 100k: 190 against 22 us).
constexpr int kFusedMinRows = 512;

bool logits_topk_via_logits(const LogitsParams& p) { return p.T < kFusedMinRows; }

size_t via_logits_bytes(const LogitsParams& p) { return align256((size_t)p.T * p.out_cols * 4); }

struct FusedLayout {
    size_t bt_s, lens_s, slog, lo, flags, counts, cand, total;
    int Ws, cols_s;
};

FusedLayout fused_layout(const LogitsParams& pf) {
    FusedLayout l{};
    const int n_pages_out = (pf.out_cols + pf.page - 1) / pf.page;
    l.Ws = (pf.W + kSampleStride - 1) / kSampleStride;
    l.cols_s = ((n_pages_out + kSampleStride - 1) / kSampleStride) * pf.page;
    size_t at = 0;
    l.bt_s = at;   at += align256((size_t)pf.B * (l.Ws > 0 ? l.Ws : 1) * 4);
    l.lens_s = at; at += align256((size_t)pf.T * 4);
    l.slog = at;   at += align256((size_t)pf.T * l.cols_s * 4);
    l.lo = at;     at += align256((size_t)pf.T * 4);
    l.flags = at;  at += align256((size_t)pf.T * 4);
    l.counts = at; at += align256((size_t)pf.T * pf.n_wchunks * 4);
    l.cand = at;   at += align256((size_t)pf.T * pf.out_cols * 8);
    l.total = at;
    return l;
}

}  // namespace

hipError_t launch_fill_empty_topk(int T, int k, int32_t* out_idx, float* out_vals, hipStream_t stream) {
    const int64_t n = (int64_t)T * k;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_empty, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, n, out_idx,
                       out_vals);
    return hipGetLastError();
}

size_t logits_topk_workspace_bytes(const LogitsParams& p, int k) {
    LogitsParams pf = p;
    if (!plan_logits(pf)) return 0;
    if (logits_topk_via_logits(p)) return via_logits_bytes(p) + align256(topk_workspace_bytes(p.T, p.out_cols, k));
    return fused_layout(pf).total;
}

hipError_t launch_logits_topk(const LogitsParams& p, int k, int32_t* out_idx, float* out_vals,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
    LogitsParams pf = p;
    if (!plan_logits(pf)) return hipErrorInvalidValue;
    if (logits_topk_via_logits(p)) {
        const size_t lb = via_logits_bytes(p);
        const size_t tb = align256(topk_workspace_bytes(p.T, p.out_cols, k));
        if (ws_bytes < lb + tb || k < 1) return hipErrorInvalidValue;
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        // the top-k's histograms start zero: the scorer clears them (no memset, and no
        // kernel of their own unless the scorer has no blocks)
        const size_t zb = topk_workspace_zero_bytes(p.T, p.out_cols, k);
        const bool scorer_runs = pf.n_wchunks > 0 && pf.n_rowblocks > 0;
        LogitsParams pl = p;
        pl.out = reinterpret_cast<float*>(ws);
        pl.out_rs = p.out_cols;
        pl.lo = nullptr;
        pl.flags = nullptr;
        pl.cand = nullptr;
        pl.counts = nullptr;
        pl.zero = zb && scorer_runs ? reinterpret_cast<uint32_t*>(ws + lb) : nullptr;
        pl.zero_words = (int)((zb + 3) / 4);  // at most 512 rows of one 16 KB histogram
        hipError_t e = launch_logits(pl, stream);
        if (e != hipSuccess) return e;
        if (zb && !scorer_runs) {
            const int64_t n = (int64_t)((zb + 3) / 4);
            hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, n,
                               reinterpret_cast<uint32_t*>(ws + lb));
        }
        TopkParams tp{};
        tp.scores = pl.out;
        tp.row_stride = p.out_cols;
        tp.rows = p.T;
        tp.cols = p.out_cols;
        tp.k = k;
        tp.row_lens = p.lens;
        tp.out_idx = out_idx;
        tp.out_vals = out_vals;
        tp.workspace = tb ? ws + lb : nullptr;
        return launch_topk(tp, stream);
    }
    if (pf.n_wchunks > kMaxChunks || k < 1 || k > kSortCap) return hipErrorInvalidValue;
    const FusedLayout l = fused_layout(pf);
    if (ws_bytes < l.total) return hipErrorInvalidValue;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* bt_s = reinterpret_cast<int32_t*>(ws + l.bt_s);
    int32_t* lens_s = reinterpret_cast<int32_t*>(ws + l.lens_s);
    float* slog = reinterpret_cast<float*>(ws + l.slog);
    float* lo = reinterpret_cast<float*>(ws + l.lo);
    int32_t* flags = reinterpret_cast<int32_t*>(ws + l.flags);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + l.counts);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws + l.cand);

    // 1. sampled table
    SampleParams sp{};
    sp.bt = p.bt;
    sp.bt_rs = p.bt_rs;
    sp.B = p.B;
    sp.W = p.W;
    sp.Ws = l.Ws;
    sp.lens = p.lens;
    sp.T = p.T;
    sp.out_cols = p.out_cols;
    sp.page = p.page;
    sp.bt_s = bt_s;
    sp.lens_s = lens_s;
    const int64_t n_items = std::max<int64_t>((int64_t)p.B * l.Ws, p.T);
    hipLaunchKernelGGL(k_sample_table, dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0, stream, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. scores of the sampled pages
    LogitsParams ps = p;
    ps.bt = bt_s;
    ps.bt_rs = l.Ws > 0 ? l.Ws : 1;
    ps.W = l.Ws;
    ps.lens = lens_s;
    ps.out = slog;
    ps.out_rs = l.cols_s;
    ps.out_cols = l.cols_s;
    ps.cand = nullptr;
    ps.lo = nullptr;
    ps.flags = nullptr;
    ps.counts = nullptr;
    if ((e = launch_logits(ps, stream)) != hipSuccess) return e;

    // 3. thresholds
    ThresholdParams tp{};
    tp.slog = slog;
    tp.lens_s = lens_s;
    tp.T = p.T;
    tp.cols_s = l.cols_s;
    tp.m = 2 * ((k + kSampleStride - 1) / kSampleStride);
    tp.lo = lo;
    hipLaunchKernelGGL(k_threshold, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0, stream, tp);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // 4. every page, keeping the scores >= lo
    pf.lo = lo;
    pf.flags = nullptr;
    pf.cand = cand;
    pf.cand_rs = pf.out_cols;
    pf.counts = counts;
    pf.counts_rs = pf.n_wchunks;
    if ((e = launch_logits(pf, stream)) != hipSuccess) return e;

    // 5. selection
    SelectParams sel{};
    sel.cand = cand;
    sel.cand_rs = pf.cand_rs;
    sel.counts = counts;
    sel.counts_rs = pf.counts_rs;
    sel.nchunks = pf.n_wchunks;
    sel.chunk_w = pf.ppw * pf.page;
    sel.lo = lo;
    sel.flags = flags;
    sel.second = 0;
    sel.T = p.T;
    sel.k = k;
    sel.out_idx = out_idx;
    sel.out_vals = out_vals;
    const size_t lds = (size_t)(pf.n_wchunks + 1) * 4;
    const dim3 sel_grid((unsigned)p.T);
    hipLaunchKernelGGL(k_fused_select, sel_grid, dim3(kSelThreads), lds, stream, sel);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // 6. flagged rows again, keeping every score
    pf.flags = flags;
    if ((e = launch_logits(pf, stream)) != hipSuccess) return e;
    sel.second = 1;
    hipLaunchKernelGGL(k_fused_select, sel_grid, dim3(kSelThreads), lds, stream, sel);
    return hipGetLastError();
}

}  // namespace fp4idx
