// topk.hip -- exact top-k selection over score rows, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Order: larger score first, ties to the smaller column; -inf and NaN are never
// selected; -0 equals +0.  Output: the selected columns in increasing order, padded
// with -1.
//
// Method: radix select on order-preserving 32-bit keys, entirely in LDS.  One
// workgroup (16 waves) takes up to 32768 elements into LDS (a row, or one chunk of a
// long row), builds 11/11/10-bit digit histograms with LDS atomics to find the exact
// threshold key T and the number of ties at T to keep, then compacts the selected
// elements in index order with wave ballots (each lane learns its output slot from the
// popcount of the lanes below it).  Rows longer than one chunk run in stages: stage 1
// keeps each chunk's own top-k (every element of the row's top-k is in its chunk's
// top-k, with the same tie rule), later stages merge up to F candidate lists per
// workgroup, and the last stage writes the result.  Lists stay in column order, so the
// final compaction is in column order as well.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxElems = 32768;          // LDS-resident elements, dense mode
constexpr int kMaxCand = kMaxElems / 2;   // candidate mode keeps keys and columns

enum Mode { kDenseFinal = 0, kDenseList = 1, kCandFinal = 2, kCandList = 3 };

// Order-preserving key: larger float -> larger key; -0 -> +0; -inf, NaN -> 0 (never
// selected: every selectable key is at least key(-FLT_MAX) = 0x00800000).
__device__ __forceinline__ uint32_t to_key(float v) {
    if (!(v > -__builtin_inff())) return 0u;
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Shared {
    uint32_t keys[kMaxElems];  // dense: keys; candidate mode: keys [0, kMaxCand), cols after
    uint32_t hist[2048];
    int wave_gt[kWaves];
    int wave_eq[kWaves];
    int list_off[9];
    int n_valid;
    uint32_t sel_digit;
    int sel_above;
};

// Find digit d (bins [0, nbins)) with above(d) < kk <= above(d) + hist[d], where
// above(d) counts the elements in bins > d.  Run by wave 0.  Writes sel_digit and
// sel_above (the count strictly above d).
__device__ void find_digit(Shared& sh, int nbins, int kk) {
    const int lane = threadIdx.x & 63;
    const int per = nbins / 64;  // 32 or 16
    int x = 0;
    for (int b = 0; b < per; b++) x += (int)sh.hist[lane * per + b];
    // inclusive suffix sum over lanes
    int s = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_down(s, d);
        if (lane + d < 64) s += y;
    }
    bool mine = (s - x < kk) && (kk <= s);
    unsigned long long m = __ballot(mine);
    int L = __ffsll((long long)m) - 1;
    if (lane == L) {
        int above = s - x;
        int d = lane * per;
        for (int b = lane * per + per - 1; b >= lane * per; b--) {
            if (above + (int)sh.hist[b] >= kk) { d = b; break; }
            above += (int)sh.hist[b];
        }
        sh.sel_digit = (uint32_t)d;
        sh.sel_above = above;
    }
}

__device__ __forceinline__ void clear_hist(Shared& sh) {
    for (int i = threadIdx.x; i < 2048; i += kThreads) sh.hist[i] = 0u;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_topk(const TopkParams p, const uint32_t* __restrict__ in_keys,
                                                   const int32_t* __restrict__ in_cols,
                                                   const int32_t* __restrict__ in_cnt, int in_lists,
                                                   uint32_t* __restrict__ out_keys, int32_t* __restrict__ out_cols,
                                                   int32_t* __restrict__ out_cnt, int out_lists, int fanout) {
    __shared__ Shared sh;
    constexpr bool kDense = MODE == kDenseFinal || MODE == kDenseList;
    constexpr bool kFinal = MODE == kDenseFinal || MODE == kCandFinal;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_groups = kDense ? p.n_chunks : out_lists;  // workgroups per row
    const int row = blockIdx.x / n_groups;
    const int grp = blockIdx.x - row * n_groups;
    if (row >= p.rows) return;
    const int k = p.k;

    uint32_t* keys = sh.keys;
    uint32_t* cols = sh.keys + kMaxCand;  // candidate mode only
    int n = 0;
    int col0 = 0;
    if constexpr (kDense) {
        int len = p.cols;
        if (p.row_lens) len = min(max(p.row_lens[row], 0), p.cols);
        col0 = grp * p.chunk;
        n = max(0, min(len - col0, p.chunk));
        const float* src = p.scores + (int64_t)row * p.row_stride + col0;
        for (int i = tid; i < n; i += kThreads) keys[i] = to_key(src[i]);
    } else {
        const int l0 = grp * fanout;
        const int l1 = min(l0 + fanout, in_lists);
        if (tid == 0) {
            int o = 0;
            for (int l = l0; l < l1; l++) {
                sh.list_off[l - l0] = o;
                o += in_cnt[(int64_t)row * in_lists + l];
            }
            sh.list_off[l1 - l0] = o;
        }
        __syncthreads();
        n = sh.list_off[l1 - l0];
        for (int l = l0; l < l1; l++) {
            const int off = sh.list_off[l - l0];
            const int cnt = sh.list_off[l - l0 + 1] - off;
            const int64_t base = ((int64_t)row * in_lists + l) * k;
            for (int i = tid; i < cnt; i += kThreads) {
                keys[off + i] = in_keys[base + i];
                cols[off + i] = (uint32_t)in_cols[base + i];
            }
        }
    }
    clear_hist(sh);
    __syncthreads();

    // ---- count valid elements and find the threshold key
    // pass 1: top 11 bits
    for (int i = tid; i < n; i += kThreads) {
        uint32_t key = keys[i];
        if (key) atomicAdd(&sh.hist[key >> 21], 1u);
    }
    __syncthreads();
    // total valid
    if (wave == 0) {
        int x = 0;
        for (int b = 0; b < 32; b++) x += (int)sh.hist[lane * 32 + b];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
        if (lane == 0) sh.n_valid = x;
    }
    __syncthreads();
    const int n_valid = sh.n_valid;
    uint32_t T;      // select key > T, plus the first `need` keys == T
    int need;
    if (n_valid <= k) {
        T = 0u;      // every valid key (> 0) is selected, no ties at 0 are kept
        need = 0;
    } else {
        if (wave == 0) find_digit(sh, 2048, k);
        __syncthreads();
        const uint32_t d1 = sh.sel_digit;
        int kk = k - sh.sel_above;
        __syncthreads();
        clear_hist(sh);
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key = keys[i];
            if (key && (key >> 21) == d1) atomicAdd(&sh.hist[(key >> 10) & 2047u], 1u);
        }
        __syncthreads();
        if (wave == 0) find_digit(sh, 2048, kk);
        __syncthreads();
        const uint32_t d2 = sh.sel_digit;
        kk -= sh.sel_above;
        __syncthreads();
        clear_hist(sh);
        __syncthreads();
        const uint32_t pre = (d1 << 11) | d2;
        for (int i = tid; i < n; i += kThreads) {
            uint32_t key = keys[i];
            if (key && (key >> 10) == pre) atomicAdd(&sh.hist[key & 1023u], 1u);
        }
        __syncthreads();
        if (wave == 0) find_digit(sh, 1024, kk);
        __syncthreads();
        T = (pre << 10) | sh.sel_digit;
        need = kk - sh.sel_above;  // >= 1 ties at T to keep
        __syncthreads();
    }

    // ---- ordered compaction: wave w owns elements [w*seg, (w+1)*seg)
    const int seg = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int e0 = wave * seg, e1 = min(e0 + seg, n);
    int gt = 0, eq = 0;
    for (int base = e0; base < e1; base += 64) {
        int i = base + lane;
        uint32_t key = i < e1 ? keys[i] : 0u;
        gt += __popcll(__ballot(key > T));
        eq += __popcll(__ballot(need > 0 && key == T));
    }
    if (lane == 0) {
        sh.wave_gt[wave] = gt;
        sh.wave_eq[wave] = eq;
    }
    __syncthreads();
    int tie_base = 0, sel_base = 0;
    for (int w = 0; w < wave; w++) {
        int e = sh.wave_eq[w];
        int take = min(max(need - tie_base, 0), e);
        sel_base += sh.wave_gt[w] + take;
        tie_base += e;
    }
    int total = 0;
    {
        int tb = 0;
        for (int w = 0; w < kWaves; w++) {
            int e = sh.wave_eq[w];
            total += sh.wave_gt[w] + min(max(need - tb, 0), e);
            tb += e;
        }
    }
    const float* srow = p.scores + (int64_t)row * p.row_stride;
    for (int base = e0; base < e1; base += 64) {
        int i = base + lane;
        uint32_t key = i < e1 ? keys[i] : 0u;
        bool is_gt = key > T;
        bool is_eq = need > 0 && key == T;
        unsigned long long mt = __ballot(is_eq);
        int tie_rank = tie_base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mt >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mt, 0u));
        bool sel = is_gt || (is_eq && tie_rank < need);
        unsigned long long ms = __ballot(sel);
        int pos = sel_base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ms >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)ms, 0u));
        if (sel) {
            int col = kDense ? col0 + i : (int)cols[i];
            if constexpr (kFinal) {
                p.out_idx[(int64_t)row * k + pos] = col;
                if (p.out_vals) p.out_vals[(int64_t)row * k + pos] = srow[col];
            } else {
                const int64_t ob = ((int64_t)row * out_lists + grp) * k;
                out_keys[ob + pos] = key;
                out_cols[ob + pos] = col;
            }
        }
        sel_base += __popcll(ms);
        tie_base += __popcll(mt);
    }
    if constexpr (kFinal) {
        for (int i = total + tid; i < k; i += kThreads) {
            p.out_idx[(int64_t)row * k + i] = -1;
            if (p.out_vals) p.out_vals[(int64_t)row * k + i] = -__builtin_inff();
        }
    } else {
        if (tid == 0) out_cnt[(int64_t)row * out_lists + grp] = total;
    }
}

// Chunk length for a row of `cols` columns: whole rows when they fit; otherwise
// chunks of 16K (few rows: more workgroups) or 32K columns.
int pick_chunk(int rows, int cols) {
    if (cols <= kMaxElems) return kMaxElems;
    return rows < 128 ? kMaxElems / 2 : kMaxElems;
}

int fanout_for(int k) { return max(2, min(8, kMaxCand / k)); }

struct WsLayout {
    int chunk, n_chunks, fanout;
    size_t list_elems;   // rows * n_chunks * k
    size_t bytes;
};

WsLayout ws_layout(int rows, int cols, int k) {
    WsLayout L{};
    L.chunk = pick_chunk(rows, cols);
    L.n_chunks = (cols + L.chunk - 1) / L.chunk;
    L.fanout = fanout_for(k);
    if (L.n_chunks <= 1) return L;
    L.list_elems = (size_t)rows * L.n_chunks * k;
    size_t one = L.list_elems * 8 + (size_t)rows * L.n_chunks * 4;
    one = (one + 255) & ~(size_t)255;
    L.bytes = 2 * one;
    return L;
}

}  // namespace

size_t topk_workspace_bytes(int rows, int cols, int k) { return ws_layout(rows, cols, k).bytes; }

hipError_t launch_topk(const TopkParams& p_in, hipStream_t stream) {
    TopkParams p = p_in;
    WsLayout L = ws_layout(p.rows, p.cols, p.k);
    p.chunk = L.chunk;
    p.n_chunks = max(1, L.n_chunks);
    const size_t smem = 0;  // static LDS (sizeof(Shared))
    if (L.n_chunks <= 1) {
        hipLaunchKernelGGL((k_topk<kDenseFinal>), dim3(p.rows), dim3(kThreads), smem, stream, p,
                           nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 1, 1);
        return hipGetLastError();
    }
    // two ping-pong list buffers in the workspace
    unsigned char* ws = reinterpret_cast<unsigned char*>(p_in.cand_vals);
    size_t one = L.bytes / 2;
    uint32_t* keys[2];
    int32_t* cols[2];
    int32_t* cnt[2];
    for (int b = 0; b < 2; b++) {
        unsigned char* base = ws + b * one;
        keys[b] = reinterpret_cast<uint32_t*>(base);
        cols[b] = reinterpret_cast<int32_t*>(base + L.list_elems * 4);
        cnt[b] = reinterpret_cast<int32_t*>(base + L.list_elems * 8);
    }
    int lists = L.n_chunks;
    hipLaunchKernelGGL((k_topk<kDenseList>), dim3((unsigned)(p.rows * lists)), dim3(kThreads), smem, stream,
                       p, nullptr, nullptr, nullptr, 0, keys[0], cols[0], cnt[0], lists, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int cur = 0;
    while (lists > L.fanout) {
        int next = (lists + L.fanout - 1) / L.fanout;
        hipLaunchKernelGGL((k_topk<kCandList>), dim3((unsigned)(p.rows * next)), dim3(kThreads), smem, stream,
                           p, keys[cur], cols[cur], cnt[cur], lists, keys[cur ^ 1], cols[cur ^ 1],
                           cnt[cur ^ 1], next, L.fanout);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        cur ^= 1;
        lists = next;
    }
    hipLaunchKernelGGL((k_topk<kCandFinal>), dim3((unsigned)p.rows), dim3(kThreads), smem, stream, p,
                       keys[cur], cols[cur], cnt[cur], lists, nullptr, nullptr, nullptr, 1, L.fanout);
    return hipGetLastError();
}

}  // namespace fp4idx
