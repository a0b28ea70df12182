// topk_stream.hip -- exact top-k of score rows, one workgroup per row streaming the
// row from memory, gfx950.
//
// ("ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Fix (production
// target)": a wave-level (ballot) top-k instead of a serial shared-memory heap merge.)
//
// Same order and output as topk.hip: larger first, ties to the smaller column, -inf
// and NaN never selected, the chosen columns in increasing order, -1 padded (values
// -inf).  Scores map to order-preserving 32-bit keys; digit 1 is key bits [31:21],
// digit 2 bits [20:10], digit 3 bits [9:0] (2048 histogram bins: 4096 took 4% longer
// on the prefill rows).
//
// One workgroup per row, no workspace and no exchange between workgroups:
//   1. sample: runs of 32 adjacent columns at evenly spaced starts, about 64 sampled
//      keys above the k-th largest key in expectation; two digit levels of their keys
//      give the 97th largest sample key (22 bits of it), `lo`, so about 1.5 k keys of
//      the row are >= lo.
//   2. stream: one pass over the row keeps every key >= lo in LDS (key and column,
//      appended in any order) and builds the exact digit-1 histogram of those keys.
//   3. the histogram and two more digit levels over the kept keys give the k-th
//      largest key K* and how many keys equal to K* are taken; every kept key above
//      K* is marked in a column bitmap, and the ties when all of them are taken.
//   4. the bitmap is read out in column order (a popcount scan) into the output row.
// Rare cases take extra passes over the row and stay exact: fewer than k keys >= lo
// (the sample overestimated lo: stream again from the lowest key), more keys >= lo
// than LDS holds (stream again keeping only keys from the k-th one's digit-1 bin, then
// its digit-2 bin, then only keys above K*), and more ties at K* than needed (two
// passes over contiguous column ranges mark the first ones in column order).
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kSBins = 2048;
constexpr int kU = 4;  // 16-byte loads per thread in one chunk of the row

__device__ __forceinline__ uint32_t skey(float v) {
    if (!(v > -__builtin_inff())) return 0u;
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of skey for selectable keys (>= skey(-FLT_MAX)).
__device__ __forceinline__ float from_skey(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// LDS layout: the histogram (uint32 words; once the last digit is settled the same
// words hold the row's column bitmap, at most 1024 words for 32768 columns), candidate
// keys (uint32), candidate columns (uint16: rows have at most 32768 columns), then a
// small area for scan totals and shared scalars.  32 KB with 4080 candidates,
// so four row workgroups share a CU.
constexpr int kStreamMaxCols = 32768;

struct StreamLds {
    uint32_t* hist;
    uint32_t* bmap;   // aliases hist
    uint32_t* ckey;
    uint16_t* ccol;
    int* wtot;   // [16] wave totals of block scans
    int* pick;   // [4] pick_bin results
    int* ctr;    // [4] candidate count
};

__device__ __forceinline__ StreamLds carve(uint32_t* lds, int cap) {
    StreamLds s;
    s.hist = lds;
    s.bmap = lds;
    s.ckey = s.hist + kSBins;
    s.ccol = reinterpret_cast<uint16_t*>(s.ckey + cap);
    s.wtot = reinterpret_cast<int*>(s.ckey + cap + cap / 2);  // cap is even
    s.pick = s.wtot + 16;
    s.ctr = s.pick + 4;
    return s;
}

size_t topk_stream_lds_bytes(int cap) { return 4 * ((size_t)kSBins + (size_t)cap + (size_t)cap / 2 + 24); }

template <int NT>
__global__ __launch_bounds__(NT) void k_topk_stream(const TopkParams p, int cap) {
    extern __shared__ __align__(16) uint32_t lds_words[];
    constexpr int NW = NT / 64;
    constexpr int PB = kSBins / NT;  // histogram bins per thread
    const StreamLds L = carve(lds_words, cap);
    // last row first: in a causal prefill rows grow with their index, so the longest
    // start first and short ones fill the kernel's tail (1.044 -> 1.012 ms at 32768 rows)
    const int row = (int)gridDim.x - 1 - (int)blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int k = p.k;
    int len = p.cols;
    if (p.row_lens) len = min(max(p.row_lens[row], 0), p.cols);
    const float* src = p.scores + (int64_t)row * p.row_stride;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)p.cols * 4u);
    const int rwords = (len + 31) / 32;  // bitmap words that cover the row

    auto clear_hist = [&]() {
#pragma unroll
        for (int b = 0; b < PB; b++) L.hist[tid + NT * b] = 0u;
    };
    // The bin holding the kk-th largest of the histogrammed keys: thread t owns bins
    // kSBins-1-PB*t .. kSBins-PB*t-PB (descending).  pick[0] = bin, [1] = keys in
    // higher bins, [2] = total, [3] = keys in the bin.  Ends with a barrier.
    // The bins are read 16 bytes at a time: with one word per read the threads' bins, PB
    // words apart, would fall into few LDS banks.
    auto pick_desc = [&](int kk) {
        int c[PB], bin[PB];
        const int lo_bin = kSBins - PB * (tid + 1);  // thread t's lowest bin (16-byte aligned)
        const v4u* hv = reinterpret_cast<const v4u*>(L.hist + lo_bin);
#pragma unroll
        for (int q = 0; q < PB / 4; q++) {
            const v4u v = hv[q];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int b = PB - 1 - (4 * q + e);  // descending: b = 0 is the highest bin
                bin[b] = lo_bin + 4 * q + e;
                c[b] = (int)v[e];
            }
        }
        pick_bin<NT, PB>(c, bin, kk, L.wtot, L.pick);
    };

    // The row streams through in chunks of kU 16-byte loads per thread (4 * NT * kU
    // columns), the next chunk's loads in flight while one is processed.  Column
    // 4 * (tid + NT * u) + e of a chunk is element e of load u.  A chunk that reaches
    // past the row end reads dwords, so no 16-byte load straddles the buffer's end.
    auto load_chunk = [&](int ch, v4f (&buf)[kU]) {
        const int cb = ch * 4 * NT * kU;
        // per-thread part of the address in a VGPR, the rest in the scalar offset
        if (cb + 4 * NT * kU <= len) {
#pragma unroll
            for (int u = 0; u < kU; u++)
                buf[u] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs, 16 * tid, 4 * cb + 16 * NT * u, 0));
        } else {
#pragma unroll
            for (int u = 0; u < kU; u++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    buf[u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                              rs, 16 * tid + 4 * e, 4 * cb + 16 * NT * u, 0));
        }
    };
    const int n_ch = (len + 4 * NT * kU - 1) / (4 * NT * kU);
    // The first pass's first two chunks are loaded while the sample is ranked (the
    // loads are issued after the sample's, so waiting for the sample leaves them in
    // flight).
    v4f ba[kU], bb[kU];
    bool pre = false;
    auto prefetch = [&]() {
        if (n_ch > 0) load_chunk(0, ba);
        if (n_ch > 1) load_chunk(1, bb);
        pre = true;
    };

    // ---- clear the histogram and the counter
    clear_hist();
    if (tid == 0) L.ctr[0] = 0;
    lds_barrier();

    // ---- 1. sample: S evenly spaced columns, about 64 of them expected above the
    // k-th largest key; lo = the first 22 bits of the rho-th largest sample key with
    // rho = 64 + 32 + 1 (four standard deviations of the sample count), so about
    // 1.5 k keys of the row are >= lo and fewer than k only with probability ~1e-4.
    // Short rows (len <= 2k) keep every valid key.
    constexpr int kSPer = 4;  // samples per thread at most
    uint32_t lo = 1u;
    if (len > 2 * k) {
        const int S = (int)min((int64_t)NT * kSPer, max((int64_t)1, ((int64_t)len * 64 + k - 1) / k));
        const int rho = 97;
        uint32_t sk[kSPer];
        // runs of 32 adjacent columns (one 128-byte line each) at evenly spaced starts
        const int runs = (S + 31) / 32;
#pragma unroll
        for (int j = 0; j < kSPer; j++) {
            const int i = tid + NT * j;
            const int c = (int)(((int64_t)(i >> 5) * len) / runs) + (i & 31);
            sk[j] = i < S ? skey(src[min(c, len - 1)]) : 0u;
        }
        prefetch();
#pragma unroll
        for (int j = 0; j < kSPer; j++)
            if (sk[j]) atomicAdd(&L.hist[sk[j] >> 21], 1u);
        lds_barrier();
        pick_desc(rho);
        if (L.pick[2] >= rho) {
            const uint32_t d1 = (uint32_t)L.pick[0];
            const int r2 = rho - L.pick[1];
            lds_barrier();
            clear_hist();
            lds_barrier();
#pragma unroll
            for (int j = 0; j < kSPer; j++)
                if (sk[j] && (sk[j] >> 21) == d1) atomicAdd(&L.hist[(sk[j] >> 10) & 0x7ffu], 1u);
            lds_barrier();
            pick_desc(r2);
            lo = (d1 << 21) | ((uint32_t)L.pick[0] << 10);
        }
        lds_barrier();
    } else {
        prefetch();
    }

    // ---- 2./3. stream passes until the kept keys settle K*
    // level 0: keep keys >= lo, histogram digit 1 of the kept keys
    // level 1: keep keys >= d1:0:0, histogram digit 2 of keys in bin d1
    // level 2: keep keys >= d1:d2:0, histogram digit 3 of keys in bin (d1, d2)
    // level 3: keep keys > K* only (fewer than k: they always fit)
    int level = 0;
    uint32_t kstar = 0u;   // K* once known
    int need = 0;          // keys equal to K* that are taken
    int ties = 0;          // keys equal to K* in the row
    int kk = k;            // rank of K* among the keys matching the current prefix
    int n_kept = 0;
    bool all_valid = false;  // fewer valid keys than k: every valid key is taken
    for (;;) {
        clear_hist();
        if (tid == 0) L.ctr[0] = 0;
        lds_barrier();
        const int hshift = level == 0 ? 21 : (level == 1 ? 10 : 0);
        const uint32_t hmask = level == 2 ? 0x3ffu : 0x7ffu;
        const int pshift = level == 0 ? 32 : (level == 1 ? 21 : 10);  // prefix bits above the digit
        const uint32_t prefix = pshift == 32 ? 0u : (lo >> pshift);
        // Kept keys go to LDS with one counter update per wave and chunk.
        // keep test in float space: key(v) >= keep_min, or key(v) > K* in level 3
        // (NaN compares false; -0 and +0 are one key and compare equal)
        const bool keep_all = level < 3 && lo <= 0x00800000u;  // every valid key
        const bool strict = level == 3 || keep_all;
        const float thr = keep_all ? -__builtin_inff() : from_skey(level == 3 ? kstar : lo);
        auto kept = [&](float v) { return strict ? v > thr : v >= thr; };
        auto process = [&](int ch, const v4f (&buf)[kU]) {
            const int cb = ch * 4 * NT * kU;
            const bool full = cb + 4 * NT * kU <= len;
            int nkeep = 0;
#pragma unroll
            for (int u = 0; u < kU; u++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    nkeep += (kept(buf[u][e]) && (full || cb + 4 * (tid + NT * u) + e < len)) ? 1 : 0;
            const int incl = wave_incl_scan(nkeep);
            const int tot = __builtin_amdgcn_readlane(incl, 63);
            if (tot == 0) return;
            int base = 0;
            if (lane == 63) base = atomicAdd(L.ctr, tot);
            base = __builtin_amdgcn_readlane(base, 63);
            int pos = base + incl - nkeep;
#pragma unroll
            for (int u = 0; u < kU; u++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int c = cb + 4 * (tid + NT * u) + e;
                    if (kept(buf[u][e]) && (full || c < len)) {
                        const uint32_t kv = skey(buf[u][e]);
                        if (level < 3 && (pshift == 32 || (kv >> pshift) == prefix))
                            atomicAdd(&L.hist[(kv >> hshift) & hmask], 1u);
                        if (pos < cap) {
                            L.ckey[pos] = kv;
                            L.ccol[pos] = (uint16_t)c;
                        }
                        pos++;
                    }
                }
        };
        // pairs of chunks alternate between two buffers; the loop body has no exit.  The
        // first pass finds chunks 0 and 1 already loaded.
        int ch = 0;
        if (n_ch > 0 && !pre) load_chunk(0, ba);
        for (; ch + 2 <= n_ch; ch += 2) {
            if (!(pre && ch == 0)) load_chunk(ch + 1, bb);
            process(ch, ba);
            if (ch + 2 < n_ch) load_chunk(ch + 2, ba);
            process(ch + 1, bb);
        }
        if (ch < n_ch) process(ch, ba);
        pre = false;
        lds_barrier();
        n_kept = L.ctr[0];
        const bool overflow = n_kept > cap;
        if (level == 3) break;  // keys above K* are all kept (fewer than k <= cap)
        pick_desc(kk);
        const int total = L.pick[2];
        if (level == 0 && total < k) {
            if (lo > 1u) {  // the sample overestimated lo: keep every valid key
                lo = 1u;
                lds_barrier();
                continue;
            }
            all_valid = true;  // fewer valid keys than k, all kept (n_kept < k <= cap)
            lds_barrier();
            break;
        }
        const uint32_t d = (uint32_t)L.pick[0];
        const int above = L.pick[1], inbin = L.pick[3];
        lds_barrier();
        if (!overflow) {
            // settle the remaining digits over the kept keys in LDS
            uint32_t pre = level == 0 ? (d << 21) : (level == 1 ? ((lo & 0xffe00000u) | (d << 10)) : ((lo & 0xfffffc00u) | d));
            int lvl = level + 1;
            kk -= above;
            ties = inbin;
            const int nk = n_kept;
            // a bin whose keys are all taken ends the digits early: K* is then its lowest
            // possible key (the prefix, low bits zero), every key at or above it is taken
            // and need == ties
            while (lvl < 3 && ties != kk) {
                clear_hist();
                lds_barrier();
                const int sh = lvl == 1 ? 10 : 0;
                const uint32_t msk = lvl == 1 ? 0x7ffu : 0x3ffu;
                const int ps = lvl == 1 ? 21 : 10;
                for (int i = tid; i < nk; i += NT) {
                    const uint32_t key = L.ckey[i];
                    if ((key >> ps) == (pre >> ps)) atomicAdd(&L.hist[(key >> sh) & msk], 1u);
                }
                lds_barrier();
                pick_desc(kk);
                const uint32_t dd = (uint32_t)L.pick[0];
                kk -= L.pick[1];
                ties = L.pick[3];
                pre |= lvl == 1 ? (dd << 10) : dd;
                lds_barrier();
                lvl++;
            }
            kstar = pre;
            need = kk;
            break;
        }
        // overflow: narrow what the next pass keeps
        kk -= above;
        if (level == 0) lo = d << 21;
        else if (level == 1) lo = (lo & 0xffe00000u) | (d << 10);
        else {
            kstar = (lo & 0xfffffc00u) | d;
            need = kk;
            ties = inbin;
        }
        level++;
    }

    // the histogram is done with: its words hold the row's column bitmap from here on
    for (int w = tid; w < rwords; w += NT) L.bmap[w] = 0u;
    lds_barrier();

    // ---- mark the selected columns
    // keys equal to K* are in LDS unless the last pass kept only keys above it
    const bool ties_kept = level < 3;
    const int nk = min(n_kept, cap);
    for (int i = tid; i < nk; i += NT) {
        const uint32_t key = L.ckey[i];
        const bool take = all_valid || key > kstar || (key == kstar && ties == need && ties_kept);
        if (take) {
            const uint32_t col = L.ccol[i];  // uint16 in LDS
            atomicOr(&L.bmap[col >> 5], 1u << (col & 31));
        }
    }
    if (!all_valid && (ties > need || !ties_kept)) {
        // the first `need` keys equal to K* in column order: wave w scans columns
        // [w*span, (w+1)*span) twice (count, then mark)
        const int span = ((len + NW - 1) / NW + 63) & ~63;
        const int cbeg = wave * span, cend = min(len, cbeg + span);
        const int steps = max(cend - cbeg + 63, 0) / 64;
        int mine = 0;
        for (int st = 0; st < steps; st++) {
            const int c = cbeg + 64 * st + lane;
            const bool eq = c < cend && skey(src[c]) == kstar;
            mine += __popcll(__ballot(eq));
        }
        if (lane == 0) L.wtot[wave] = mine;
        lds_barrier();
        int before = 0;
        for (int w = 0; w < wave; w++) before += L.wtot[w];
        for (int st = 0; st < steps; st++) {
            const int c = cbeg + 64 * st + lane;
            const bool eq = c < cend && skey(src[c]) == kstar;
            const unsigned long long m = __ballot(eq);
            const int r = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (eq && r < need) atomicOr(&L.bmap[c >> 5], 1u << (c & 31));
            before += __popcll(m);
        }
    }
    lds_barrier();

    // ---- 4. the bitmap in column order: thread t owns words [t*WPT, (t+1)*WPT)
    const int wpt = (rwords + NT - 1) / NT;
    int cnt = 0;
    for (int j = 0; j < wpt; j++) {
        const int w = tid * wpt + j;
        if (w < rwords) cnt += __popc(L.bmap[w]);
    }
    int excl, total;
    block_excl_scan<NT>(cnt, L.wtot, excl, total);
    int32_t* oi = p.out_idx + (int64_t)row * k;
    float* ov = p.out_vals ? p.out_vals + (int64_t)row * k : nullptr;
    int pos = excl;
    for (int j = 0; j < wpt; j++) {
        const int w = tid * wpt + j;
        if (w >= rwords) break;
        uint32_t bits = L.bmap[w];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            const int col = 32 * w + b;
            if (pos < k) {
                oi[pos] = col;
                if (ov) ov[pos] = src[col];
            }
            pos++;
        }
    }
    for (int i = total + tid; i < k; i += NT) {
        oi[i] = -1;
        if (ov) ov[i] = -__builtin_inff();
    }
}

}  // namespace

// Candidates kept in LDS: k plus slack (at least k, which the exact fallbacks need).
// With k plus about 2000 the LDS stays within 32 KB, so four row workgroups share a CU
// with room to spare (the waves' registers allow four; a fifth by a register cap
// measured no faster): 4080 candidates for k = 2048; larger k take up to 150 KB.
int topk_stream_cap(int cols, int k) {
    if (cols > kStreamMaxCols || k < 1) return -1;
    const size_t fixed = topk_stream_lds_bytes(0);
    auto room = [&](size_t budget) { return budget > fixed ? (int)(((budget - fixed) / 6) & ~(size_t)1) : 0; };
    const int want = k + 2048;
    const int cap32 = room(32u * 1024u);
    int cap = want <= cap32 + 16 ? (want < cap32 ? want : cap32) : (want < room(150u * 1024u) ? want : room(150u * 1024u));
    cap &= ~1;
    return cap < k ? -1 : cap;
}

hipError_t launch_topk_stream(const TopkParams& p, hipStream_t stream) {
    const int cap = topk_stream_cap(p.cols, p.k);
    if (cap < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_topk_stream<256>, dim3(p.rows), dim3(256), topk_stream_lds_bytes(cap), stream, p, cap);
    return hipGetLastError();
}

}  // namespace fp4idx
