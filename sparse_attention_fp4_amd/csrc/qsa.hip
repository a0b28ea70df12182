// qsa.hip -- sparse attention over the tokens a top-k selection names, reading an fp8
// (e4m3fn) paged K/V cache, gfx950.
//
// (vLLM qsa_fp8 API page: _qsa_physical_slots_kernel, _decode_slot_layout,
// _qsa_sparse_paged_decode_kernel and qsa_sparse_paged_decode.)
//
// Slot pass: one thread per (row, column) turns a logical token into
// (physical page << offset_bits) | place, or -1 when the request, the token, its logical
// page or its physical page is out of range.  It runs once per row for every KV head.
//
// Decode: one workgroup of four waves per (row, KV head).  The row's selected columns
// are cut into chunks of 32; wave w takes chunks w, w+4, ... and keeps its own online
// softmax (running max, partial sum, 16 heads x 128 dims of fp32 output); the four
// partial states are merged through LDS at the end.  Per chunk:
//   * scores S^T[32 tokens x 16 heads] = K Q^T on V_MFMA_F32_16X16X32_BF16: K rows are
//     gathered as 32-byte pieces (four lanes per 128-byte row) and converted exactly
//     from e4m3fn to bf16 in registers; q is bf16 as given.  Token rows are assigned to
//     the two 16-row tiles so that each lane ends up holding the scores of 8 consecutive
//     tokens of one head (the page multiplies the same exact bf16 products).
//   * p = exp2(s * scale * log2 e - running max), rounded to fp16 for the product (as
//     the page does); the partial sum uses the fp32 values.
//   * O^T[128 dims x 16 heads] += V^T P^T on V_MFMA_F32_16X16X32_F16.  Each lane
//     gathers 8 bytes (8 dims) of each of its 8 tokens' V rows; a byte permute and the
//     packed e4m3fn->fp16 conversion turn them into the transposed operand (one dim,
//     8 tokens) without an LDS round trip.  MFMA c covers dims 8n + c (n = 0..15), so a
//     lane's 32 accumulators are 32 consecutive dims of one head.
// Loads are unconditional: a token that is not selected (column past the valid count,
// slot -1, a page or place outside the cache) reads page 0 of its head instead, its score is
// masked and its V bytes are zeroed, so every address stays inside the cache.
// Epilogue as the page: output_scale / sum, rounded to bf16, times sigmoid(gate),
// rounded to bf16; a row with no selected token writes zeros.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kQsaWaves = 4;
constexpr int kQsaThreads = 64 * kQsaWaves;
constexpr int kChunk = 32;
constexpr int kDim = 128;
constexpr int kORow = kDim + 4;  // LDS row of a wave's partial output (padded)
constexpr float kMaskedMax = -1e30f;
constexpr int kSeg = 4096;       // columns whose token offsets are staged in LDS at a time

__global__ __launch_bounds__(256) void k_qsa_slots(const QsaSlotParams p, int col_blocks) {
    const int r = blockIdx.x / col_blocks;
    const int c = (blockIdx.x - r * col_blocks) * 256 + threadIdx.x;
    if (c >= p.slot_cols) return;
    int32_t slot = -1;
    const int b = p.t2r[r];
    if (c < p.topk && b >= 0 && b < p.num_req) {
        const int32_t x = p.ind[(int64_t)r * p.ind_rs + c];
        if (x >= 0) {
            const int lp = x / p.page;
            if (lp < p.width) {
                const int32_t pg = p.bt[(int64_t)b * p.bt_rs + lp];
                if (pg >= 0 && pg < p.num_blocks)
                    slot = (int32_t)(((uint32_t)pg << p.ob) | (uint32_t)(x - lp * p.page));
            }
        }
    }
    p.slots[(int64_t)r * p.slots_rs + c] = slot;
}

__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 e4m3fn codes (code i in byte i % 4 of word i / 4) -> 8 bf16, exact.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// e4m3fn codes in bytes 0,1 (HI = false) or 2,3 (HI = true) of w -> two fp16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const v2h h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const v2h h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// One chunk's gathered bytes for one lane.
struct QsaRaw {
    uint4 k[2][2];   // K tile j: 32 bytes (dims 32*qg .. +32) of tile row (lane & 15)
    uint2 v[8];      // V: 8 bytes (dims 8*(lane & 15) .. +8) of token 8*qg + i
    uint32_t valid;  // bit i: token 8*qg + i is selected
};

__global__ __launch_bounds__(kQsaThreads) void k_qsa_decode(const QsaDecodeParams p) {
    // LDS: the byte offsets of one segment of columns while the chunks run (bit 0 set
    // for a selected token), the waves' partial outputs for the final merge
    union QsaLds {
        uint64_t off[kSeg];
        float o[kQsaWaves][16][kORow];
    };
    __shared__ QsaLds lds;
    __shared__ float s_m[kQsaWaves][16];
    __shared__ float s_l[kQsaWaves][16];

    const int r = blockIdx.x / p.Hkv;
    const int g = blockIdx.x - r * p.Hkv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hn = lane & 15;  // MFMA row/column index: head of the group, tile row, dim/8
    const int qg = lane >> 4;  // lane group: tokens 8*qg .. 8*qg+7 of a chunk

    int n = p.ind[(int64_t)r * p.ind_rs + p.topk];
    n = __builtin_amdgcn_readfirstlane(min(max(n, 0), p.topk));

    // q operand of k-step s: dims 32*qg + 8*s .. +8 of head g*G + hn (zero past the group)
    v8bf qop[4];
    {
        const uint16_t* qrow = p.q + (int64_t)r * p.q_rs + (int64_t)(g * p.G + hn) * p.q_hs + 32 * qg;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            uint4 t = make_uint4(0, 0, 0, 0);
            if (hn < p.G) t = *(const uint4*)(qrow + 8 * s);
            qop[s] = __builtin_bit_cast(v8bf, t);
        }
    }

    const int32_t* srow = p.slots + (int64_t)r * p.slots_rs;
    const uint8_t* kbase = p.k + (int64_t)g * p.khs + 32 * qg;
    const uint8_t* vbase = p.v + (int64_t)g * p.vhs + 8 * hn;
    const uint32_t omask = (1u << p.ob) - 1u;
    const uint32_t bs = (uint32_t)p.bs, ts = (uint32_t)p.ts;

    // gather the chunk's K and V pieces of this lane; a token that is not selected
    // (offset 0, bit 0 clear) reads page 0, place 0
    auto fetch = [&](int ch, QsaRaw& raw) {
        const uint64_t* so = lds.off + ch * kChunk;
        raw.valid = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint64_t off = so[8 * qg + i];
            raw.v[i] = *(const uint2*)(vbase + (off & ~(uint64_t)1));
            raw.valid |= ((uint32_t)off & 1u) << i;
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            // tile j row hn holds token 8*(hn/4) + 4*j + hn%4: its scores land in lane
            // group hn/4 as that group's tokens 4*j .. 4*j+3
            const uint64_t off = so[8 * (hn >> 2) + 4 * j + (hn & 3)];
            const uint4* kp = (const uint4*)(kbase + (off & ~(uint64_t)1));
            raw.k[j][0] = kp[0];
            raw.k[j][1] = kp[1];
        }
    };

    float m = kMaskedMax, l = 0.f;
    v4f acc[8];
#pragma unroll
    for (int c = 0; c < 8; c++) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

    // one chunk: scores, online softmax, P V
    auto process = [&](const QsaRaw& cur) {
        // scores of tokens 8*qg + 4*j + i for head hn
        float x[8];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const uint32_t* kw = (const uint32_t*)&cur.k[j][0];
            v4f sc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++)
                sc = mfma_bf16_16x16x32(e4m3x8_to_bf16(kw[2 * s], kw[2 * s + 1]), qop[s], sc);
#pragma unroll
            for (int i = 0; i < 4; i++) x[4 * j + i] = sc[i] * p.score_scale;
        }
        float cm = kMaskedMax;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            x[t] = (cur.valid >> t) & 1u ? x[t] : kMaskedMax;
            cm = fmaxf(cm, x[t]);
        }
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float mn = fmaxf(m, cm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float pr[8], ps = 0.f;
#pragma unroll
        for (int t = 0; t < 8; t++) {
            pr[t] = (cur.valid >> t) & 1u ? __builtin_amdgcn_exp2f(x[t] - mn) : 0.f;
            ps += pr[t];
        }
        l = l * alpha + ps;
        m = mn;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int c = 0; c < 8; c++) acc[c] *= alpha;
        }
        v4u pop;
#pragma unroll
        for (int k = 0; k < 4; k++) pop[k] = pack_f16x2(pr[2 * k], pr[2 * k + 1]);
        const v8h pB = __builtin_bit_cast(v8h, pop);

        // V of unselected tokens is zeroed (its bytes may be anything)
        uint2 vv[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const bool ok = (cur.valid >> i) & 1u;
            vv[i].x = ok ? cur.v[i].x : 0u;
            vv[i].y = ok ? cur.v[i].y : 0u;
        }
#pragma unroll
        for (int cp = 0; cp < 4; cp++) {
            // dims 8*hn + 2*cp and + 1: byte (2*cp) % 4 and the next of word cp / 2
            const uint32_t sel = (cp & 1) ? 0x07030602u : 0x05010400u;
            v4u a0, a1;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t w0 = (cp >> 1) ? vv[2 * k].y : vv[2 * k].x;
                const uint32_t w1 = (cp >> 1) ? vv[2 * k + 1].y : vv[2 * k + 1].x;
                // bytes: [w0.b, w1.b, w0.b+1, w1.b+1]
                const uint32_t w = __builtin_amdgcn_perm(w1, w0, sel);
                a0[k] = e4m3x2_to_f16x2<false>(w);
                a1[k] = e4m3x2_to_f16x2<true>(w);
            }
            acc[2 * cp] = mfma_f16_16x16x32(__builtin_bit_cast(v8h, a0), pB, acc[2 * cp]);
            acc[2 * cp + 1] = mfma_f16_16x16x32(__builtin_bit_cast(v8h, a1), pB, acc[2 * cp + 1]);
        }
    };

    for (int seg0 = 0; seg0 < n; seg0 += kSeg) {
        const int ns = min(kSeg, n - seg0);
        const int nch = (ns + kChunk - 1) / kChunk;
        __syncthreads();  // the previous segment's offsets are no longer read
        // byte offset of each column's token row, bit 0 set when it is selected: the
        // slot is not -1 and its page and place lie inside the cache (-1 gives a page
        // past the cache); columns past the segment's count are not selected
        // (loads clamped to the last column so that they all issue before the first wait)
        constexpr int kPer = kSeg / kQsaThreads;
        uint32_t sl[kPer];
#pragma unroll
        for (int u = 0; u < kPer; u++)
            sl[u] = (uint32_t)srow[seg0 + min((int)threadIdx.x + u * kQsaThreads, ns - 1)];
#pragma unroll
        for (int u = 0; u < kPer; u++) {
            const int c = threadIdx.x + u * kQsaThreads;
            const uint32_t pg = sl[u] >> p.ob, pl = sl[u] & omask;
            const bool ok = c < ns && pg < (uint32_t)p.num_blocks && pl < (uint32_t)p.page;
            const uint64_t o = ((uint64_t)pg * bs + (uint64_t)pl * ts) | 1u;
            if (c < nch * kChunk) lds.off[c] = ok ? o : 0ull;
        }
        __syncthreads();
        if (wave >= nch) continue;
        // this wave's chunks wave, wave+4, ...: two buffers in turn, the next chunk's
        // gathers in flight while one is processed (no copies between them, no exit
        // inside the loop body)
        const int K = (nch - wave + kQsaWaves - 1) / kQsaWaves;
        QsaRaw A, B;
        fetch(wave, A);
        int k = 0;
        for (; k + 2 <= K; k += 2) {
            fetch(wave + (k + 1) * kQsaWaves, B);
            __builtin_amdgcn_sched_barrier(0);  // B's gathers go out before A is waited on
            process(A);
            fetch(wave + min(k + 2, K - 1) * kQsaWaves, A);  // the last one re-reads a chunk
            __builtin_amdgcn_sched_barrier(0);
            process(B);
        }
        if (k < K) process(A);
    }

    // merge the four waves' states
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // the offsets are no longer read: the LDS takes the partial outputs
    if (qg == 0) {
        s_m[wave][hn] = m;
        s_l[wave][hn] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        // accumulator c, element i: dim 8*(4*qg + i) + c of head hn
        float* o = &lds.o[wave][hn][32 * qg + 8 * i];
        *(float4*)o = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
        *(float4*)(o + 4) = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
    }
    __syncthreads();

    const int h = threadIdx.x >> 4;         // head of the group
    const int d0 = (threadIdx.x & 15) * 8;  // 8 dims
    if (h >= p.G) return;
    float M = kMaskedMax;
#pragma unroll
    for (int w = 0; w < kQsaWaves; w++) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kQsaWaves; w++) {
        const float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
        L += s_l[w][h] * f;
        const float4 a = *(const float4*)&lds.o[w][h][d0];
        const float4 b = *(const float4*)&lds.o[w][h][d0 + 4];
        o[0] += a.x * f; o[1] += a.y * f; o[2] += a.z * f; o[3] += a.w * f;
        o[4] += b.x * f; o[5] += b.y * f; o[6] += b.z * f; o[7] += b.w * f;
    }
    const float inv = p.out_scale / fmaxf(L, 1e-20f);
    const int64_t hq = (int64_t)g * p.G + h;
    const uint4 gw = *(const uint4*)(p.gate + (int64_t)r * p.gate_rs + hq * p.gate_hs + d0);
    const uint32_t gb[4] = {gw.x, gw.y, gw.z, gw.w};
    uint32_t ob[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t pair = 0;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const float gv = bf16_value((gb[k] >> (16 * e)) & 0xffffu);
            const float sig = 1.f / (1.f + __expf(-gv));
            const float y = L > 0.f ? o[2 * k + e] * inv : 0.f;
            const float z = bf16_value(bf16_rne(y)) * sig;
            pair |= bf16_rne(z) << (16 * e);
        }
        ob[k] = pair;
    }
    *(uint4*)(p.out + (int64_t)r * p.out_rs + hq * p.out_hs + d0) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
}

}  // namespace

hipError_t launch_qsa_slots(const QsaSlotParams& p, hipStream_t stream) {
    if (p.rows == 0 || p.slot_cols == 0) return hipSuccess;
    const int col_blocks = (p.slot_cols + 255) / 256;
    hipLaunchKernelGGL(k_qsa_slots, dim3((unsigned)(p.rows * col_blocks)), dim3(256), 0, stream, p,
                       col_blocks);
    return hipGetLastError();
}

hipError_t launch_qsa_decode(const QsaDecodeParams& p, hipStream_t stream) {
    if (p.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(k_qsa_decode, dim3((unsigned)(p.rows * p.Hkv)), dim3(kQsaThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp4idx
