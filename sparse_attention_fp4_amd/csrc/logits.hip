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
// or 1); the columns [0, out_cols) are cut into chunks of `ppw` key pages.  A
// workgroup takes one row block and four consecutive column chunks (one per wave), so
// the grid covers the whole [T, out_cols] output exactly once.  The workgroup first
// copies the row block's A operands (packed queries and their scale codes, or the
// decoded NVFP4 values) into LDS in the order the lanes read them, and the head weights
// next to them; each wave keeps its weights in registers and reads one A tile at a
// time from LDS, so a wave holds few registers and three waves share each SIMD.
//
// MFMA mapping.  The contraction is [rows*heads x 128] x [128 x 16 keys].  A-tile j
// holds 16 (row, head) pairs arranged so that output lane group g = l/16 always sees
// the same query row: tile row m = 4*g' + i stands for row t0 + g' % RG and head
// (16/RG)*jj + 4*(g'/RG) + i of key head hk (j = hk * tiles_per_kv + jj).  After the
// epilogue each lane therefore holds partial head sums of one (row, key) pair; with
// RG < 4 the 4/RG lane groups of a row are added with cross-lane steps.
//
// Keys go straight from HBM into the B operand, in 64-token slabs (see the slab
// section below for which lane reads which bytes); each key byte is used by exactly one
// wave, so keys skip LDS on this path.  A wave walks its pages slab by slab with the
// loads of the next two slabs in flight while it computes one; the block-table entries
// of its pages come in with one load per 64 pages.  Pages past the end of every row
// of the block get -inf without any key traffic, and a workgroup that has no visible
// page at all skips the operand staging.
//
// Rounding.  MXFP4: one scaled MFMA per (tile, key head) covers all 128 products.
// NVFP4: E2M1 x E4M3 is not an MX operand, so both sides are decoded exactly to fp16
// (value = E2M1 * 2^a * b, at most 6 significant bits) and four fp16 MFMAs accumulate
// in fp32.  Head sums use four accumulators per lane (chains of at most 8 fused
// multiply-adds: one per A tile) and a tree, so each term meets at most 8 + 2 (+ 2
// cross-lane) roundings, about 7e-7 of sum_h |w_h ReLU(dot_h)| in the worst case,
// inside the 1e-6 bound.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

constexpr int kWavesMultiRow = 4;  // waves per workgroup sharing a row block of 2 or 4 rows
constexpr int kWavesOneRow = 2;    // with one row per block (batched decode: 77.5 -> 75.6 us)
constexpr int waves_per_block(int rows_per_block) {
    return rows_per_block == 1 ? kWavesOneRow : kWavesMultiRow;
}
constexpr int kTargetWaves = 16384;    // waves of one launch (8192 .. 65536 measured)
constexpr int kTargetWavesOneRequest = 1600;  // with a single request (see plan_logits)
constexpr int kPipe = 2;               // products in flight in the epilogue pipeline
constexpr int kMaxTiles = 16;          // A tiles per block at most (8 or 16)
constexpr int kMaxPagesPerWave = 128;  // pages per wave at most (a multiple of 64)

// ---------------------------------------------------------------- operand types
template <int FMT>
struct Operand;
template <>
struct Operand<0> {  // MXFP4: raw nibbles and one E8M0 code
    v4i v;
    int s;
};
template <>
struct Operand<1> {  // NVFP4: 32 exact fp16 values in four MFMA chunks
    v8h v[4];
};

struct RawTile {     // 16 bytes of nibbles + the scale bytes that cover them
    v4i v;
    uint32_t s;
};

// Lane l's 16 bytes hold elements [32*(l/16), +32).  MXFP4: one E8M0 code for them.
// NVFP4: two E4M3 codes (groups 2*(l/16) and 2*(l/16)+1); dword c of the bytes (chunk
// c of the fp16 MFMA) lies in group 2*(l/16) + c/2.
template <int FMT>
__device__ __forceinline__ Operand<FMT> decode(const RawTile& r) {
    Operand<FMT> o;
    if constexpr (FMT == 0) {
        o.v = r.v;
        o.s = (int)r.s;
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            float pw, bb;
            e4m3_split((r.s >> (8 * (c >> 1))) & 0xffu, pw, bb);
            o.v[c] = decode8_f16((uint32_t)r.v[c], pw, bb);
        }
    }
    return o;
}

template <int FMT>
__device__ __forceinline__ v4f tile_dot(const Operand<FMT>& a, const Operand<FMT>& b) {
    if constexpr (FMT == 0) {
        return mfma_fp4_16x16x128(a.v, a.s, b.v, b.s, v4f{0.f, 0.f, 0.f, 0.f});
    } else {
        v4f d = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; c++) d = mfma_f16_16x16x32(a.v[c], b.v[c], d);
        return d;
    }
}

// Scale bytes of one 128-value query vector that lane group g needs.
template <int FMT>
__device__ __forceinline__ uint32_t scale_bytes(const uint8_t* s, int g) {
    if constexpr (FMT == 0) return s[g];
    else return (uint32_t)s[2 * g] | ((uint32_t)s[2 * g + 1] << 8);
}

// ReLU of a per-head dot.  NVFP4: fmaxf (IEEE maxNum: a NaN dot, which only a NaN E4M3
// scale code can make, counts as 0).  MXFP4: one integer max on the bit pattern (every
// negative value, -0 included, becomes +0; positive values pass), which saves the
// quieting step fmaxf needs on a matrix-core result.  An MXFP4 dot is NaN only for
// E8M0 scale code 255, which the format never stores; such a NaN passes through.
template <int FMT>
__device__ __forceinline__ float relu(float d) {
    if constexpr (FMT == 0) return __int_as_float(max(__float_as_int(d), 0));
    else return fmaxf(d, 0.0f);
}

// Cross-lane sum of the 4/RG lane groups that share a row.
template <int RG>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (RG == 1) {
        v = add_lane_xor16(v);
        v = add_lane_xor32(v);
    } else if constexpr (RG == 2) {
        v = add_lane_xor32(v);
    }
    return v;
}

// ---------------------------------------------------------------- key slabs
// A slab is 64 consecutive tokens of one key head of one page.  Column n of MFMA tile
// tt (tt = 0..3) is token 4n + tt of the slab, so lane (g, n) reads bytes [16g, +16)
// of tokens 4n .. 4n+3 (four loads at 64-byte steps), the scale bytes of those four
// tokens in one 16-byte (MXFP4) or two (NVFP4) loads, and ends up holding the logits
// of four adjacent columns, which it writes with one 16-byte store.
//
// Loads go through buffer descriptors built per slab in scalar registers (base =
// the slab's first byte).  A slab that does not exist or whose page is invisible or
// invalid gets a descriptor of zero bytes: its loads return zeros without touching
// memory, so every slab issues the same instructions and no branch separates a load
// from its use.
template <int FMT>
struct Slab {
    v4i k[4];                    // tile tt: bytes [16g, +16) of token 4n + tt
    v4i s[FMT == 0 ? 1 : 2];     // the scale bytes of tokens 4n .. 4n+3
};

// Scale operand of tile tt from the slab's scale bytes.  MXFP4: byte 4tt + g (the
// E8M0 code of elements [32g, +32) of token 4n + tt).  NVFP4: the E4M3 codes of groups
// 2g and 2g+1 of that token, bytes 8tt + 2g and 8tt + 2g + 1, as a 16-bit pair.
template <int FMT>
__device__ __forceinline__ uint32_t slab_scale(const Slab<FMT>& b, int tt, int g) {
    if constexpr (FMT == 0) {
        return ((uint32_t)b.s[0][tt] >> (8 * g)) & 0xffu;
    } else {
        const int dw = 2 * tt + (g >> 1);
        const uint32_t word = (uint32_t)b.s[dw >> 2][dw & 3];
        return (word >> (16 * (g & 1))) & 0xffffu;
    }
}

// ---------------------------------------------------------------- A operands in LDS
// The workgroup's A operands live in LDS for the whole kernel, stored in the order the
// lanes read them, so a tile costs one conflict-free read per lane and no registers
// between uses:
//   MXFP4: slot (j, l) = lane l's 16 bytes of nibbles of A tile j ([NT][64] x 16 B), and
//          the E8M0 codes of all tiles of lane l side by side ([64][NT] bytes), so one
//          read gives a lane every code; the MFMA takes tile j's byte through its
//          operand-select field.
//   NVFP4: the decoded fp16 operand in four 16-byte chunks ([NT][4][64] x 16 B).
// The head weights follow in the order the epilogue applies them: [NT][4][4] floats,
// entry (j, g, i) = the weight of tile row 4g + i of A tile j (0 for padding rows), so
// lane group g reads its four weights of a tile as one 16-byte broadcast.
template <int FMT, int NT>
struct ALayout {
    static constexpr int kOpBytes = FMT == 0 ? 16 : 64;
    static constexpr int kScaleOff = NT * 64 * kOpBytes;
    static constexpr int kWOff = kScaleOff + (FMT == 0 ? NT * 64 : 0);
    static constexpr size_t kBytes = (size_t)kWOff + NT * 64;
};

// A row held by slot (j, l): row offset `toff` in the row block and head `h`, with the
// 16 bytes it needs at [16 * (l / 16), +16).  False for padding slots (heads past the
// key head's count or tiles past n_tiles).
template <int RG>
__device__ __forceinline__ bool slot_row(const LogitsParams& p, int j, int l, int& toff, int& h) {
    const int m = l & 15, gp = m >> 2, i0 = m & 3;
    const int hk = j / p.tiles_per_kv, jj = j - hk * p.tiles_per_kv;
    const int hl = (16 / RG) * jj + 4 * (gp / RG) + i0;
    toff = gp % RG;
    h = hk * p.R + hl;
    return j < p.n_tiles && hl < p.R;
}

constexpr uint32_t kOffNone = 0x80000000u;  // buffer offset past every output range
constexpr int kNonTemporal = 2;              // cache-policy bit of a streaming store

template <int FMT, int SEL>
__device__ __forceinline__ v4f tile_dot_sel(const Operand<FMT>& a, uint32_t a_codes,
                                            const Operand<FMT>& b) {
    if constexpr (FMT == 0) {
        const v8i A = {a.v[0], a.v[1], a.v[2], a.v[3], 0, 0, 0, 0};
        const v8i B = {b.v[0], b.v[1], b.v[2], b.v[3], 0, 0, 0, 0};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4,
                                                                SEL, (int)a_codes, 0, b.s);
    } else {
        (void)a_codes;
        return tile_dot<FMT>(a, b);
    }
}

// ---------------------------------------------------------------- the kernel
// MKV: more than one key head (the tiles of key head hk only meet that head's slabs).
// FUSE: the scores are not stored; those at or above the row's threshold are kept as
// top-k candidates (see LogitsParams).
template <int FMT, int RG, int NT, bool MKV, bool FUSE>
// MXFP4 16-tile blocks that store their scores (prefill) are held to four waves per SIMD
// (128 registers, a few spilled outside the slab loop).  The fused variant and smaller
// blocks keep their registers: there the spills cost more than the extra wave gains.
__global__ __launch_bounds__(64 * waves_per_block(RG))
__attribute__((amdgpu_waves_per_eu(FMT == 0 && NT == 16 && !FUSE ? 4 : 1, 8))) void k_logits(const LogitsParams p) {
    constexpr int kWavesPerBlock = waves_per_block(RG);
    constexpr int kThreads = 64 * kWavesPerBlock;
    extern __shared__ __align__(16) uint8_t lds[];
    using L = ALayout<FMT, NT>;
    constexpr int G = FMT == 0 ? 4 : 8;
    uint8_t* sa = lds;                                          // operands, lane order
    uint8_t* sac = lds + L::kScaleOff;                          // MXFP4 codes [64][NT]
    float* sw = reinterpret_cast<float*>(lds + L::kWOff);       // weights [NT][4][4]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar math
    const int g = lane >> 4, n = lane & 15;
    const int bq = blockIdx.x / p.n_wgchunks;
    const int wc = (blockIdx.x - bq * p.n_wgchunks) * kWavesPerBlock + wave;
    const int t0 = bq * RG;
    const int nrows = min(RG, p.T - t0);
    const int t_last = t0 + nrows - 1;
    if constexpr (FUSE) {
        // second pass of the fused top-k: only row blocks holding a flagged row
        if (p.flags) {
            bool any = false;
            for (int i = 0; i < nrows; i++) any = any || p.flags[t0 + i] != 0;
            if (!any) return;
        }
    }

    const int n_pages_out = (p.out_cols + p.page - 1) / p.page;
    const int lp_begin = wc * p.ppw;
    const int lp_end = min(lp_begin + p.ppw, n_pages_out);
    const bool has_work = wc < p.n_wchunks;
    const int halves = p.page / 64;
    const int slabs_per_page = halves * p.Hkv;
    const int t_out = t0 + (g % RG);
    const int koff = 256 * n + 16 * g;          // lane's byte offset in a slab's keys
    const int soff = 4 * G * n;                 // and in its scale bytes
    const bool lane_stores = g < RG;            // lane groups that hold a row's final sums

    // ---- output.  Lane (g, n) with g < RG writes columns col0 .. col0+3 (col0 = the
    // slab's first column + 4n) of row t0 + g.  Stores go through a descriptor based at
    // the slab's first column of row t0 (the host keeps (RG-1) rows + 64 columns within
    // 2^31 bytes); lanes that must not store get an offset past its range, so every
    // slab issues the same store instructions without a branch.  Streaming
    // (non-temporal): the logits are not read again by this kernel, and keeping them
    // out of L2 leaves room for the keys.  A slab inside the output takes one 16-byte
    // store per lane, the last one of a row four 4-byte stores.
    const int64_t row_base = (int64_t)t0 * p.out_rs;
    const uint32_t lane_off = (uint32_t)(((int64_t)(g % RG) * p.out_rs + 4 * n) * 4);
    const uint32_t out_range = (uint32_t)(((int64_t)(RG - 1) * p.out_rs + 64) * 4);
    auto store_slab = [&](int colb, const float (&o)[4], bool st) {
        const int col0 = colb + 4 * n;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + row_base + colb, out_range);
        if (colb + 64 <= p.out_cols) {
            const v4f ov = v4f{o[0], o[1], o[2], o[3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, ov), ro,
                                                   st ? lane_off : kOffNone, 0, kNonTemporal);
        } else {
#pragma unroll
            for (int tt = 0; tt < 4; tt++)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(o[tt]), ro, st && col0 + tt < p.out_cols ? lane_off + 4u * tt : kOffNone,
                    0, kNonTemporal);
        }
    };
    // -inf over the wave's pages [pi0, lp_end - lp_begin): no keys are read there
    // (nothing to keep when fused)
    auto fill = [&](int pi0, bool st) {
        if constexpr (FUSE) return;
        const float ninf[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
        for (int pi = pi0; pi < lp_end - lp_begin; pi++)
            for (int hf = 0; hf < halves; hf++) store_slab((lp_begin + pi) * p.page + hf * 64, ninf, st);
    };
    // ---- fused top-k candidates.  Lane (g, n) keeps those of its four scores that
    // reach its row's threshold; ballots give every kept score its rank among the
    // group's kept scores of the slab (column order), and the group's running count
    // `run` places the slab after the earlier ones of the wave's chunk.  Stores go
    // through a descriptor at row t0's candidates; a score not kept gets an offset past
    // its range.
    float lo_t = 0.f;
    if constexpr (FUSE) {
        const int tl = t0 + min(g % RG, max(nrows, 1) - 1);
        lo_t = p.lo[tl];
        if (p.flags && p.flags[tl] != 0) lo_t = -__builtin_inff();
    }
    const int64_t cand_c0 = (int64_t)lp_begin * p.page;  // the chunk's first column
    const uint32_t cand_range = (uint32_t)(((int64_t)(RG - 1) * p.cand_rs + p.out_cols) * 8);
    auto append = [&](int colb, const float (&o)[4], bool st, int& run) {
        bool kp[4];
#pragma unroll
        for (int tt = 0; tt < 4; tt++) kp[tt] = st && o[tt] >= lo_t && o[tt] > -__builtin_inff();
        const uint64_t gmask = 0xffffull << (16 * g);
        const uint64_t below = gmask & ((1ull << lane) - 1ull);
        int pre = 0, tot = 0;
#pragma unroll
        for (int tt = 0; tt < 4; tt++) {
            const uint64_t b = __ballot(kp[tt]);
            pre += __popcll(b & below);
            tot += __popcll(b & gmask);
        }
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.cand + (int64_t)t0 * p.cand_rs, cand_range);
        const int64_t base = (int64_t)(g % RG) * p.cand_rs + cand_c0 + run + pre;
        int j = 0;
#pragma unroll
        for (int tt = 0; tt < 4; tt++) {
            const uint64_t e = (uint64_t)__float_as_uint(o[tt]) | ((uint64_t)(uint32_t)(colb + 4 * n + tt) << 32);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, e), rc,
                                                  kp[tt] ? (uint32_t)((base + j) * 8) : kOffNone, 0, 0);
            j += kp[tt] ? 1 : 0;
        }
        run += tot;
    };

    // ---- prologue.  Loads go out in the order their results are needed: the first
    // segment's metadata (request, row lengths, block-table entries), then the
    // workgroup's A operands and weights, then the first two key slabs.  The LDS stores
    // of the operands wait only for their loads and the barrier only for LDS, so the key
    // loads stay in flight across both.  Lane i of my_phys[w] holds the physical page of
    // page lp_begin + 64w + i (-1: invisible or invalid); with one request the
    // block-table row is known without the request lookup.
    // Every prologue load reads a valid address (indices are clamped into range) and the
    // unwanted values are replaced afterwards, so no branch separates a load from its use
    // and each wait covers just the loads it needs.
    RowRequest rq = find_request(p.cu, p.B, t0);
    const int nr1 = max(nrows, 1);  // a row block always holds at least one row
    const int lens_raw = p.lens[t0 + min(g % RG, nr1 - 1)];
    constexpr int kWin = (kMaxPagesPerWave + 63) / 64;  // 64-page windows per wave
    int bt_raw[kWin];  // the block-table entry of page lp_begin + 64w + lane (clamped)
#pragma unroll
    for (int w = 0; w < kWin; w++) {
        bt_raw[w] = -1;
        if (has_work && p.W > 0) {
            const int b_first = p.B == 1 ? 0 : rq.b;
            bt_raw[w] = p.bt[(int64_t)b_first * p.bt_rs + min(lp_begin + 64 * w + lane, p.W - 1)];
        }
    }
    // operand slots of this thread: the query bytes and scale codes of each
    constexpr int kSlots = (NT * 64 + kThreads - 1) / kThreads;
    constexpr int kSW = (NT * 16 + kThreads - 1) / kThreads;  // NT * 16 weights
    v4i st_q[kSlots];
    uint32_t st_s[kSlots];
    bool st_ok[kSlots];
    float st_w[kSW];
    bool stw_ok[kSW];
#pragma unroll
    for (int k = 0; k < kSlots; k++) {
        const int slot = threadIdx.x + kThreads * k;
        const int j = slot >> 6, l = slot & 63;
        int toff, h;
        const bool ok = slot < NT * 64 && slot_row<RG>(p, j, l, toff, h) && toff < nrows;
        st_ok[k] = ok;
        const int t = t0 + (ok ? toff : 0), hh = ok ? h : 0, c = l >> 4;
        st_q[k] = load16(p.q + (int64_t)t * p.q_rs + hh * 64 + 16 * c);
        st_s[k] = scale_bytes<FMT>(p.qs + (int64_t)t * p.qs_rs + hh * G, c);
    }
#pragma unroll
    for (int k = 0; k < kSW; k++) {
        // weight entry (j, gg, ii): row t0 + gg % RG, head of tile row 4 gg + ii
        const int i = threadIdx.x + kThreads * k;
        const int j = i >> 4, gg = (i >> 2) & 3, ii = i & 3;
        const int hk = j / p.tiles_per_kv, jj = j - hk * p.tiles_per_kv;
        const int hlo = (16 / RG) * jj + 4 * (gg / RG) + ii, to = gg % RG;
        const bool ok = i < NT * 16 && j < p.n_tiles && hlo < p.R && to < nrows;
        stw_ok[k] = ok;
        st_w[k] = p.w[(int64_t)(t0 + (ok ? to : 0)) * p.w_rs + (ok ? hk * p.R + hlo : 0)];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (p.zero) {  // this workgroup's share of a region to clear, after its own loads
        const int w0 = blockIdx.x * p.zero_per_block, w1 = min(w0 + p.zero_per_block, p.zero_words);
        for (int w = w0 + threadIdx.x; w < w1; w += kThreads) p.zero[w] = 0u;
    }
    // A workgroup whose columns all lie past every row's end only writes -inf (all its
    // waves see the same rows, so they all leave here or none does).
    {
        const int lr = (g % RG) < nrows ? min(lens_raw, p.out_cols) : 0;
        const int wg_max = uniform(max_lane_xor32i(max_lane_xor16i(lr)));
        const int wg_col0 = (blockIdx.x - bq * p.n_wgchunks) * kWavesPerBlock * p.ppw * p.page;
        if (wg_col0 >= wg_max) {
            if (has_work) fill(0, lane_stores && g < nrows);
            if constexpr (FUSE) {
                if (has_work && n == 0 && lane_stores && g < nrows)
                    p.counts[(int64_t)(t0 + g) * p.counts_rs + wc] = 0;
            }
            return;
        }
    }
    int b = 0, seg_end = t0, len = 0, my_phys[kWin];
    int vis_pages = 0, n_vis = 0;  // the wave's pages (slabs) before every row's end
    bool row_ok = false;
    auto setup_segment = [&](int t_seg, bool first) {
        if (!first) rq = find_request(p.cu, p.B, t_seg);
        b = rq.b;
        const bool req_ok = rq.ok;
        seg_end = req_ok ? min(rq.end, t_last + 1) : t_last + 1;
        row_ok = t_out >= t_seg && t_out < seg_end;
        const int lens_pref = (g % RG) < nrows ? lens_raw : 0;
        len = (row_ok && req_ok) ? min(lens_pref, p.out_cols) : 0;
        const int max_len = uniform(max_lane_xor32i(max_lane_xor16i(len)));
#pragma unroll
        for (int w = 0; w < kWin; w++) {
            my_phys[w] = -1;
            const int lp = lp_begin + 64 * w + lane;
            if (has_work && req_ok && lp < lp_end && lp * p.page < max_len && lp < p.W) {
                const int v = first ? bt_raw[w] : p.bt[(int64_t)b * p.bt_rs + lp];
                my_phys[w] = (v >= 0 && v < p.num_pages) ? v : -1;
            }
        }
        vis_pages = has_work ? min(max((max_len + p.page - 1) / p.page - lp_begin, 0), lp_end - lp_begin) : 0;
        n_vis = vis_pages * slabs_per_page;
    };
    // physical page of the wave's page pi (wave-uniform)
    auto phys_of = [&](int pi) {
        int ph = __builtin_amdgcn_readlane(my_phys[0], pi & 63);
#pragma unroll
        for (int w = 1; w < kWin; w++)
            if ((pi >> 6) == w) ph = __builtin_amdgcn_readlane(my_phys[w], pi & 63);
        return ph;
    };
    // slab s of this wave: page lp_begin + pi, half `half` of it, key head hk (fastest)
    // (one key head: a page holds one or two slabs, so shifts replace the division)
    auto slab_pos = [&](int s, int& pi, int& half, int& hk) {
        if constexpr (!MKV) {
            const int sh = halves - 1;
            pi = s >> sh, half = s & sh, hk = 0;
        } else {
            pi = s / slabs_per_page;
            const int r = s - pi * slabs_per_page;
            half = r / p.Hkv;
            hk = r - half * p.Hkv;
        }
    };
    // Branch-free: a slab that is not there reads page 0 through a zero-byte descriptor.
    auto issue = [&](int s, Slab<FMT>& dst) {
        int pi, half, hk;
        slab_pos(s, pi, half, hk);
        const int phys = phys_of(pi);
        const bool ok = s < n_vis && phys >= 0;
        const int64_t pg = ok ? phys : 0;
        const int64_t tok = (int64_t)hk * p.page + half * 64;
        const uint8_t* kb = p.k + pg * p.kp_s + tok * 64;
        const uint8_t* sb = p.ks + pg * p.ksp_s + tok * G;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, ok ? 64u * 64u : 0u);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sb, ok ? 64u * G : 0u);
#pragma unroll
        for (int tt = 0; tt < 4; tt++)
            dst.k[tt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * tt, 0, 0));
#pragma unroll
        for (int c = 0; c < (FMT == 0 ? 1 : 2); c++)
            dst.s[c] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, soff + 16 * c, 0, 0));
    };
    Slab<FMT> b0, b1;
    setup_segment(t0, true);
    issue(0, b0);
    issue(1, b1);
    __builtin_amdgcn_sched_barrier(0);

    // ---- operands and weights into LDS (zeros in padding slots and past T)
#pragma unroll
    for (int k = 0; k < kSlots; k++) {
        const int slot = threadIdx.x + kThreads * k;
        if (slot < NT * 64) {
            const int j = slot >> 6, l = slot & 63;
            RawTile r;
            r.v = st_ok[k] ? st_q[k] : v4i{0, 0, 0, 0};
            r.s = st_ok[k] ? st_s[k] : (FMT == 0 ? 127u : 0u);
            if constexpr (FMT == 0) {
                *reinterpret_cast<v4i*>(sa + (size_t)slot * 16) = r.v;
                sac[l * NT + j] = (uint8_t)r.s;
            } else {
                const Operand<1> o = decode<1>(r);
#pragma unroll
                for (int c = 0; c < 4; c++)
                    *reinterpret_cast<v8h*>(sa + ((size_t)(j * 4 + c) * 64 + l) * 16) = o.v[c];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kSW; k++) {
        const int i = threadIdx.x + kThreads * k;
        if (i < NT * 16) sw[i] = stw_ok[k] ? st_w[k] : 0.0f;
    }
    lds_barrier();
    if (!has_work) return;  // uniform per wave, after the only barrier

    // ---- per-lane head weights (lane group g sums rows 4g .. 4g+3 of each tile) and
    // MXFP4 scale codes; neither depends on the request segment: a lane only ever adds
    // products of its own query row
    auto w_tile = [&](int j) { return *reinterpret_cast<const v4f*>(sw + (j * 4 + g) * 4); };
    // more than 8 tiles: the weights are read from LDS a tile at a time
    constexpr bool kWLds = NT > 8;
    v4f wv[kWLds ? 1 : NT];
    if constexpr (!kWLds) {
#pragma unroll
        for (int j = 0; j < NT; j++) wv[j] = w_tile(j);
    }
    uint32_t acodes[(NT + 3) / 4];
    if constexpr (FMT == 0) {
        if constexpr (NT == 16) {
            const uint4 c4 = *reinterpret_cast<const uint4*>(sac + lane * NT);
            acodes[0] = c4.x, acodes[1] = c4.y, acodes[2] = c4.z, acodes[3] = c4.w;
        } else if constexpr (NT == 8) {
            const uint2 c2 = *reinterpret_cast<const uint2*>(sac + lane * NT);
            acodes[0] = c2.x, acodes[1] = c2.y;
        } else if constexpr (NT == 4) {
            acodes[0] = *reinterpret_cast<const uint32_t*>(sac + lane * NT);
        } else {
            acodes[0] = *reinterpret_cast<const uint16_t*>(sac + lane * NT);
        }
    } else {
#pragma unroll
        for (int i = 0; i < (NT + 3) / 4; i++) acodes[i] = 0;
    }
    auto a_op = [&](int j) {
        Operand<FMT> o;
        if constexpr (FMT == 0) {
            o.v = *reinterpret_cast<const v4i*>(sa + ((size_t)j * 64 + lane) * 16);
            o.s = 0;
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++)
                o.v[c] = *reinterpret_cast<const v8h*>(sa + ((size_t)(j * 4 + c) * 64 + lane) * 16);
        }
        return o;
    };

    // The rows of a block may belong to different requests; each pass handles the rows
    // of one request (rows of a request are consecutive).
    int t_seg = t0;
    while (t_seg <= t_last) {
        if (t_seg != t0) {
            setup_segment(t_seg, false);
            issue(0, b0);
            issue(1, b1);
        }
        const bool st_lane = lane_stores && row_ok;
        int run = 0;  // kept candidates of this lane's row in the chunk (fused)
        // ---- the wave's slabs: two buffers in turn (the next slab's keys are in flight
        // while one is computed; a third measured slower)
        // head sums: acc[set][key tile][i]; tiles 8*set .. 8*set+7 go to one set, so
        // no accumulation chain is longer than 8 multiply-adds
        constexpr int kSets = NT > 8 ? 2 : 1;
        float acc[kSets][4][4];
#pragma unroll
        for (int c = 0; c < kSets; c++)
#pragma unroll
            for (int tt = 0; tt < 4; tt++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[c][tt][i] = 0.0f;
        Operand<FMT> acur = a_op(0);  // the A tile the next product needs
        v4f wcur = v4f{0.f, 0.f, 0.f, 0.f}, wnext = v4f{0.f, 0.f, 0.f, 0.f};
        if constexpr (kWLds) wnext = w_tile(0);  // weights of the epilogue's tile, the next
        auto compute = [&](int s, const Slab<FMT>& buf) {
            int pi, half, hk;
            slab_pos(s, pi, half, hk);
            const int phys = phys_of(pi);
            const bool last_kv = !MKV || hk == p.Hkv - 1;  // all key heads of these keys are in
            const int col0 = (lp_begin + pi) * p.page + half * 64 + 4 * n;
            float o[4];
            if (phys >= 0) {
                Operand<FMT> kb[4];
#pragma unroll
                for (int tt = 0; tt < 4; tt++) {
                    RawTile rt;
                    rt.v = buf.k[tt];
                    rt.s = slab_scale<FMT>(buf, tt, g);
                    kb[tt] = decode<FMT>(rt);
                }
                // Products q = 4j + tt (A tile j outer, key tile tt inner), software
                // pipelined: the matrix core computes product q while the vector ALU
                // applies ReLU and the head weights to product q-(DEPTH-1).  A tile
                // j+1 (wrapping to tile 0 of the next slab) is read from LDS while tile
                // j is in use.  Scheduling barriers keep that order (left alone, the
                // compiler puts each product's epilogue right behind it and the wave
                // waits for every product in turn).
                constexpr int NP = 4 * NT;
                constexpr int DEPTH = kPipe;  // products in flight
                v4f dq[DEPTH];
                Operand<FMT> anext = acur;
#pragma unroll
                for (int q = 0; q < NP + DEPTH - 1; q++) {
                    if (q < NP) {
                        const int j = q >> 2, tt = q & 3;
                        if (tt == 0) anext = a_op(j + 1 < NT ? j + 1 : 0);
                        v4f d = v4f{0.f, 0.f, 0.f, 0.f};
                        if (!MKV || j / p.tiles_per_kv == hk) {
                            switch (j & 3) {
                                case 0: d = tile_dot_sel<FMT, 0>(acur, acodes[j >> 2], kb[tt]); break;
                                case 1: d = tile_dot_sel<FMT, 1>(acur, acodes[j >> 2], kb[tt]); break;
                                case 2: d = tile_dot_sel<FMT, 2>(acur, acodes[j >> 2], kb[tt]); break;
                                default: d = tile_dot_sel<FMT, 3>(acur, acodes[j >> 2], kb[tt]); break;
                            }
                        }
                        dq[q % DEPTH] = d;
                        if (tt == 3) acur = anext;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const int qp = q - (DEPTH - 1);
                    if (qp >= 0) {
                        const int jp = qp >> 2, tp = qp & 3;
                        v4f wj;
                        if constexpr (kWLds) {
                            // tile jp's weights were read four products ago; read the
                            // next tile's (wrapping to the next slab's first) now
                            if (tp == 0) {
                                wcur = wnext;
                                wnext = w_tile(jp + 1 < NT ? jp + 1 : 0);
                            }
                            wj = wcur;
                        } else {
                            wj = wv[kWLds ? 0 : jp];
                        }
                        if (!MKV || jp / p.tiles_per_kv == hk) {
                            // four independent ReLUs first, then the four multiply-adds,
                            // so no instruction waits on the one just before it; without
                            // key heads the first tile starts the sums (one multiply
                            // instead of zeroing them after every store)
                            const v4f d = dq[qp % DEPTH];
                            float r[4];
#pragma unroll
                            for (int i = 0; i < 4; i++) r[i] = relu<FMT>(d[i]);
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                acc[jp >> 3][tp][i] = (!MKV && (jp & 7) == 0)
                                                          ? wj[i] * r[i]
                                                          : __builtin_fmaf(wj[i], r[i], acc[jp >> 3][tp][i]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (!last_kv) return;
#pragma unroll
                for (int tt = 0; tt < 4; tt++) {
                    float v = (acc[0][tt][0] + acc[0][tt][1]) + (acc[0][tt][2] + acc[0][tt][3]);
                    if constexpr (kSets == 2)
                        v += (acc[1][tt][0] + acc[1][tt][1]) + (acc[1][tt][2] + acc[1][tt][3]);
                    v = group_sum<RG>(v);
                    o[tt] = col0 + tt < len ? v : -__builtin_inff();
                }
                if constexpr (MKV) {
#pragma unroll
                    for (int c = 0; c < kSets; c++)
#pragma unroll
                        for (int tt = 0; tt < 4; tt++)
#pragma unroll
                            for (int i = 0; i < 4; i++) acc[c][tt][i] = 0.0f;
                }
            } else {
                // an invisible page (past every row's length, or invalid) only gets -inf
                if (!last_kv) return;
#pragma unroll
                for (int tt = 0; tt < 4; tt++) o[tt] = -__builtin_inff();
            }
            if constexpr (FUSE) append(col0 - 4 * n, o, st_lane, run);
            else store_slab(col0 - 4 * n, o, st_lane);
        };
        // The loop body has no early exit: the last one or two slabs are computed
        // after it.  (An exit taken in the middle of the body would join the loop
        // head and make the wait counters there assume that the latest slab must be
        // in, which drains the ring once per pass.)
        int s = 0;
        for (; s + 2 <= n_vis; s += 2) {
            compute(s, b0);
            issue(s + 2, b0);
            compute(s + 1, b1);
            issue(s + 3, b1);
        }
        if (s < n_vis) compute(s, b0);
        fill(vis_pages, st_lane);
        if constexpr (FUSE) {
            if (st_lane && n == 0) p.counts[(int64_t)t_out * p.counts_rs + wc] = run;
        }
        t_seg = seg_end;
    }
}
template <int FMT, int RG, int NT, bool FUSE>
hipError_t launch4(const LogitsParams& p_in, hipStream_t stream) {
    LogitsParams p = p_in;
    const int64_t blocks = (int64_t)p.n_rowblocks * p.n_wgchunks;
    if (blocks <= 0) return hipSuccess;
    if (p.zero) p.zero_per_block = (int)((p.zero_words + blocks - 1) / blocks);
    const size_t lds = ALayout<FMT, NT>::kBytes;
    const dim3 threads(64 * waves_per_block(RG));
    if (p.Hkv == 1)
        hipLaunchKernelGGL((k_logits<FMT, RG, NT, false, FUSE>), dim3((unsigned)blocks), threads, lds, stream, p);
    else
        hipLaunchKernelGGL((k_logits<FMT, RG, NT, true, FUSE>), dim3((unsigned)blocks), threads, lds, stream, p);
    return hipGetLastError();
}

template <int FMT, int RG, int NT>
hipError_t launch3(const LogitsParams& p, hipStream_t stream) {
    return p.cand ? launch4<FMT, RG, NT, true>(p, stream) : launch4<FMT, RG, NT, false>(p, stream);
}

template <int FMT, int RG>
hipError_t launch2(const LogitsParams& p, hipStream_t stream) {
    if (p.n_tiles <= 2) return launch3<FMT, RG, 2>(p, stream);
    if (p.n_tiles <= 4) return launch3<FMT, RG, 4>(p, stream);
    if constexpr (RG > 1) {  // one row per block never needs more than 8 tiles (H <= 128)
        if (p.n_tiles > 8) return launch3<FMT, RG, 16>(p, stream);
    }
    return launch3<FMT, RG, 8>(p, stream);
}

template <int FMT>
hipError_t launch1(const LogitsParams& p, hipStream_t stream) {
    switch (p.rows_per_block) {
        case 4: return launch2<FMT, 4>(p, stream);
        case 2: return launch2<FMT, 2>(p, stream);
        default: return launch2<FMT, 1>(p, stream);
    }
}

}  // namespace

bool plan_logits(LogitsParams& p) {
    // Rows per A-tile group: as many as the average request holds (up to 4), reduced
    // while the block would need more than kMaxTiles A tiles (at most 16;
    // they live in LDS).  Any choice is correct; rows of different requests in one block
    // are handled in separate passes.
    int rg = 1;
    if (p.T >= 4 * p.B) rg = 4;
    else if (p.T >= 2 * p.B) rg = 2;
    for (;;) {
        const int hpt = 16 / rg;  // heads per A tile per row
        p.tiles_per_kv = (p.R + hpt - 1) / hpt;
        p.n_tiles = p.Hkv * p.tiles_per_kv;
        if (p.n_tiles <= kMaxTiles || rg == 1) break;
        rg >>= 1;
    }
    if (p.n_tiles > 8 * (rg == 1 ? 1 : 2)) return false;  // H <= 128 is checked by the caller
    p.rows_per_block = rg;
    p.n_rowblocks = (p.T + rg - 1) / rg;
    const int n_pages_out = (p.out_cols + p.page - 1) / p.page;
    // pages per wave: about kTargetWaves waves, at most kMaxPagesPerWave
    // pages each.  Long waves spread the per-workgroup set-up (operand staging, the
    // first key loads) over more work; enough of them keep every SIMD busy.  A single
    // request's rows (decode verify rows) have few pages and are latency-bound: about
    // one round of waves does best there (4 rows x 400k keys: 12.4 us with 4 pages a
    // wave, 15.0 with 1, 13.7 with 8; 100k keys: 1 page a wave).  Pages past every
    // row's end only get -inf, from a loop that reads no keys.
    const int64_t total = (int64_t)p.n_rowblocks * n_pages_out;
    const int64_t target = p.B == 1 ? kTargetWavesOneRequest : kTargetWaves;
    int64_t ppw = (total + target - 1) / target;
    ppw = ppw < 1 ? 1 : (ppw > kMaxPagesPerWave ? kMaxPagesPerWave : ppw);
    p.ppw = (int)ppw;
    p.n_wchunks = (n_pages_out + p.ppw - 1) / p.ppw;
    const int wpb = waves_per_block(rg);
    p.n_wgchunks = (p.n_wchunks + wpb - 1) / wpb;
    return true;
}

hipError_t launch_logits(const LogitsParams& p_in, hipStream_t stream) {
    LogitsParams p = p_in;
    if (!plan_logits(p)) return hipErrorInvalidValue;
    if (p.n_wchunks == 0 || p.n_rowblocks == 0) return hipSuccess;
    return p.fmt == 0 ? launch1<0>(p, stream) : launch1<1>(p, stream);
}

}  // namespace fp4idx
