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
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kSampleStride = 16;   // one logical page in 16 is scored first
constexpr int kSelThreads = 256;
constexpr int kMaxChunks = 8192;    // column chunks per row (the scorer's plan stays below)
constexpr int kStageCap = 6144;     // kept entries of a row staged in LDS
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

// block-wide helpers for 256 threads
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}

// One wave finds, in a 256-bin histogram, the digit where the count from the top
// reaches `want` (bins read from LDS; lane l owns bins 255-4l .. 252-4l).
__device__ __forceinline__ void pick_digit(const int* hist, int want, int& digit, int& above) {
    const int lane = threadIdx.x & 63;
    int c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        c[i] = hist[255 - 4 * lane - i];
        s += c[i];
    }
    const int incl = wave_incl_scan(s);  // keys in bins >= 252 - 4 lane
    const int excl = incl - s;
    const unsigned long long hit = __ballot(incl >= want && excl < want);
    const int src = hit ? __ffsll((long long)hit) - 1 : 63;
    int d = 0, a = 0;
    if (lane == src) {
        int run = excl;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (run + c[i] >= want) {
                d = 255 - 4 * lane - i;
                a = run;
                break;
            }
            run += c[i];
        }
    }
    digit = __shfl(d, src);
    above = __shfl(a, src);
}

struct ThresholdParams {
    const float* slog;   // [T][cols_s]
    const int32_t* lens_s;
    int T, cols_s, m;
    float* lo;           // [T]
};

// lo of each row: one wave per row, four digit passes over its sampled scores.
__global__ __launch_bounds__(256) void k_threshold(const ThresholdParams p) {
    __shared__ int hist[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= p.T) return;  // whole wave: no block barrier below
    int* h = hist[wave];
    const float* row = p.slog + (int64_t)t * p.cols_s;
    const int S = max(0, min(p.lens_s[t], p.cols_s));
    uint32_t prefix = 0, mask = 0;
    int want = p.m;
    bool enough = true;
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int i = 0; i < 4; i++) h[lane * 4 + i] = 0;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (int c = lane; c < S; c += 64) {
            const float v = row[c];
            if (!(v > -__builtin_inff())) continue;  // -inf and NaN are never chosen
            const uint32_t key = order_key(__float_as_uint(v));
            if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (pass == 0) {
            int tot = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) tot += h[lane * 4 + i];
            tot = wave_incl_scan(tot);
            if (__shfl(tot, 63) < want) {
                enough = false;
                break;
            }
        }
        int digit, above;
        pick_digit(h, want, digit, above);
        want -= above;
        prefix |= (uint32_t)digit << shift;
        mask |= 255u << shift;
        __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) p.lo[t] = enough ? __uint_as_float(key_value_bits(prefix)) : -__builtin_inff();
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
    int ent_off, sel_off;   // dynamic LDS: entry staging and sorting buffers (bytes)
    int P;                  // sorting network width (power of two >= k, >= 64)
};

// Dynamic LDS of the selection: 256 histogram bins, 8 scalars, the prefix of the chunk
// counts (nchunks + 1 ints), kStageCap staged entries, P sorting slots.
constexpr int kSelPreOff = (256 + 8) * 4;

// Exact top-k of one row's kept entries: one 256-lane workgroup per row.
__global__ __launch_bounds__(kSelThreads) void k_fused_select(const SelectParams p) {
    extern __shared__ __align__(16) uint8_t smem[];
    struct {
        int* hist;
        int* misc;
        int* pre;
        uint64_t* ent;
    } L = {reinterpret_cast<int*>(smem), reinterpret_cast<int*>(smem) + 256,
           reinterpret_cast<int*>(smem + kSelPreOff), reinterpret_cast<uint64_t*>(smem + p.ent_off)};
    uint64_t* const sel = reinterpret_cast<uint64_t*>(smem + p.sel_off);
    const int t = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (p.second && p.flags[t] == 0) return;  // uniform

    // ---- prefix of the chunk counts
    const int nch = p.nchunks;
    const int32_t* cnt = p.counts + (int64_t)t * p.counts_rs;
    constexpr int kPer = (kMaxChunks + kSelThreads - 1) / kSelThreads;
    int loc[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        const int c = tid * kPer + i;
        loc[i] = c < nch ? cnt[c] : 0;
        sum += loc[i];
    }
    int incl = wave_incl_scan(sum);
    if (lane == 63) L.misc[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; w++) wbase += L.misc[w];
    const int N = L.misc[0] + L.misc[1] + L.misc[2] + L.misc[3];
    int run = wbase + incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        const int c = tid * kPer + i;
        if (c < nch) L.pre[c] = run;
        run += loc[i];
    }
    if (tid == 0) L.pre[nch] = N;
    const float lo_t = p.second ? -__builtin_inff() : p.lo[t];
    if (!p.second) {
        const bool flag = lo_t > -__builtin_inff() && N < p.k;
        if (tid == 0) p.flags[t] = flag ? 1 : 0;
        if (flag) return;  // uniform
    }
    __syncthreads();

    const uint64_t* crow = p.cand + (int64_t)t * p.cand_rs;
    auto fetch = [&](int i) -> uint64_t {  // entry i of the row (chunk by binary search)
        int a = 0, b = nch;  // pre[a] <= i < pre[b]
        while (b - a > 1) {
            const int mid = (a + b) >> 1;
            if (L.pre[mid] <= i) a = mid;
            else b = mid;
        }
        return crow[(int64_t)a * p.chunk_w + (i - L.pre[a])];
    };
    const bool staged = N <= kStageCap;
    if (staged) {
        for (int i = tid; i < N; i += kSelThreads) L.ent[i] = fetch(i);
        __syncthreads();
    }
    auto ent = [&](int i) -> uint64_t { return staged ? L.ent[i] : fetch(i); };
    auto key_of = [](uint64_t e) { return order_key((uint32_t)e); };

    // ---- the k-th largest key (all entries are chosen when there are at most k)
    uint32_t kth = 0;
    int rest = N;        // entries equal to kth that are chosen
    int32_t col_cut = 0x7fffffff;
    if (N > p.k) {
        uint32_t prefix = 0, mask = 0;
        int want = p.k;
        for (int pass = 0; pass < 4; pass++) {
            const int shift = 24 - 8 * pass;
            L.hist[tid] = 0;
            __syncthreads();
            for (int i = tid; i < N; i += kSelThreads) {
                const uint32_t key = key_of(ent(i));
                if ((key & mask) == prefix) atomicAdd(&L.hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            int digit = 0, above = 0;
            if (wave == 0) {
                pick_digit(L.hist, want, digit, above);
                if (lane == 0) L.misc[4] = digit, L.misc[5] = above;
            }
            __syncthreads();
            digit = L.misc[4];
            above = L.misc[5];
            want -= above;
            prefix |= (uint32_t)digit << shift;
            mask |= 255u << shift;
            __syncthreads();
        }
        kth = prefix;
        rest = want;
        // ties at the k-th key: the `rest` smallest columns among them
        if (tid == 0) L.misc[6] = 0;
        __syncthreads();
        int eq = 0;
        for (int i = tid; i < N; i += kSelThreads) eq += key_of(ent(i)) == kth ? 1 : 0;
        atomicAdd(&L.misc[6], eq);
        __syncthreads();
        const int n_eq = L.misc[6];
        __syncthreads();
        if (n_eq > rest) {
            int a = 0, b = 0x7fffffff;  // the smallest c with #(tied columns <= c) >= rest
            while (a < b) {
                const int mid = a + ((b - a) >> 1);
                if (tid == 0) L.misc[7] = 0;
                __syncthreads();
                int c = 0;
                for (int i = tid; i < N; i += kSelThreads) {
                    const uint64_t e = ent(i);
                    c += (key_of(e) == kth && (int32_t)(e >> 32) <= mid) ? 1 : 0;
                }
                atomicAdd(&L.misc[7], c);
                __syncthreads();
                if (L.misc[7] >= rest) b = mid;
                else a = mid + 1;
                __syncthreads();
            }
            col_cut = a;
        }
    }

    // ---- the chosen entries, sorted by column (bitonic network over a power of two)
    const int m = min(N, p.k);
    const int P = p.P;
    if (tid == 0) L.misc[4] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kSelThreads) {
        const uint64_t e = ent(i);
        const uint32_t key = key_of(e);
        const bool take = N <= p.k || key > kth || (key == kth && (int32_t)(e >> 32) <= col_cut);
        if (take) {
            const int at = atomicAdd(&L.misc[4], 1);
            // sort key: column in the high half
            if (at < P) sel[at] = e;
        }
    }
    __syncthreads();
    for (int i = m + tid; i < P; i += kSelThreads) sel[i] = ~0ull;  // sorts last
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P; i += kSelThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const uint64_t a = sel[i], b = sel[j];
                    const bool up = (i & size) == 0;
                    const bool sw = up ? ((a >> 32) > (b >> 32)) : ((a >> 32) < (b >> 32));
                    if (sw) {
                        sel[i] = b;
                        sel[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    int32_t* oi = p.out_idx + (int64_t)t * p.k;
    float* ov = p.out_vals ? p.out_vals + (int64_t)t * p.k : nullptr;
    for (int i = tid; i < p.k; i += kSelThreads) {
        const bool ok = i < m;
        const uint64_t e = ok ? sel[i] : 0ull;
        oi[i] = ok ? (int32_t)(e >> 32) : -1;
        if (ov) ov[i] = ok ? __uint_as_float((uint32_t)e) : -__builtin_inff();
    }
}

__global__ __launch_bounds__(256) void k_fill_empty(int64_t n, int32_t* idx, float* vals) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    idx[i] = -1;
    if (vals) vals[i] = -__builtin_inff();
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
    (void)k;
    LogitsParams pf = p;
    if (!plan_logits(pf)) return 0;
    return fused_layout(pf).total;
}

hipError_t launch_logits_topk(const LogitsParams& p, int k, int32_t* out_idx, float* out_vals,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
    LogitsParams pf = p;
    if (!plan_logits(pf)) return hipErrorInvalidValue;
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
    int P = 64;
    while (P < k) P <<= 1;
    sel.P = P;
    sel.ent_off = (kSelPreOff + (pf.n_wchunks + 1) * 4 + 15) & ~15;
    sel.sel_off = sel.ent_off + kStageCap * 8;
    const size_t lds = (size_t)sel.sel_off + (size_t)P * 8;
    hipLaunchKernelGGL(k_fused_select, dim3((unsigned)p.T), dim3(kSelThreads), lds, stream, sel);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // 6. flagged rows again, keeping every score
    pf.flags = flags;
    if ((e = launch_logits(pf, stream)) != hipSuccess) return e;
    sel.second = 1;
    hipLaunchKernelGGL(k_fused_select, dim3((unsigned)p.T), dim3(kSelThreads), lds, stream, sel);
    return hipGetLastError();
}

}  // namespace fp4idx
