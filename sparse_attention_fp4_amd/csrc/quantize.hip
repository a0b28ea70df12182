// quantize.hip -- MXFP4 quantize-and-store of index keys into the paged cache, gfx950.
//
// ("[DSv4.1] Speed up the FP4 indexer scorer...", Modifications and the bench: bf16
// keys are stored as E2M1 nibbles plus one E8M0 code per 32 values, rounded to nearest
// even, at the page and token their slot names, with exponent codes clamped to
// 1..254; "ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", "Why it's
// wrong": the nibble is the index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.)
//
// Block exponent (not given on the pages; the OCP microscaling rule): scale =
// 2^(floor(log2(amax)) - 2), so amax / scale lies in [4, 8); code = that exponent + 127
// clamped to 1..254.  For a normal amax the biased fp32 exponent field is
// floor(log2(amax)) + 127, so code = field - 2; zero and subnormal maxima give code 1.
//
// Four tokens per wave, 16 lanes a token: lane j of a token holds elements 8j .. 8j+7
// (one 16-byte load of eight bf16), so the 4 lanes j = 4b .. 4b+3 hold block b and its
// maximum is a reduction over a DPP quad.  Lane j writes the 4 bytes of its 8 nibbles
// (a token's 64 bytes in one coalesced 16-lane store) and lane 4b writes block b's code.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

// Maximum over the 4 lanes of each DPP quad (values are non-negative float bit
// patterns, whose unsigned order is their numeric order).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));  // lane ^ 1
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));  // lane ^ 2
    return v;
}

// Magnitude m >= 0 (already divided by the block scale) -> index of the nearest level,
// ties to the even index; above 6 -> 6.  The index counts the midpoints between levels
// that m passes; at a midpoint the comparison (strict or not) picks the even
// neighbour, and NaN passes none (index 0).  Branch-free: seven compares.
__device__ __forceinline__ uint32_t e2m1_index_rne(float m) {
    return (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +  // 0.5 | 1 (0.75, 1.25 -> 1)
           (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) +                          // 1.5 | 2 (1.75, 2.5 -> 2)
           (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);                            // 3 | 4 (3.5, 5 -> 4) | 6
}

__device__ __forceinline__ uint32_t nibble(float x, int code) {
    const float q = __builtin_ldexpf(x, 127 - code);  // exact: a power-of-two scale
    return e2m1_index_rne(__builtin_fabsf(q)) | ((__float_as_uint(x) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void k_quantize_store(const QuantParams p) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;                                     // lane within the token
    const int n = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool in = n < p.N;
    const int nn = in ? n : p.N - 1;                             // loads stay in range
    const int64_t slot = p.slots[nn];
    const uint16_t* src = p.keys + (int64_t)nn * p.key_rs + 8 * j;  // 4-byte aligned
    uint4 raw;
    if (p.keys_aligned16) {
        raw = *reinterpret_cast<const uint4*>(src);
    } else {
        const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src);
        raw = make_uint4(s4[0], s4[1], s4[2], s4[3]);
    }
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    uint32_t a = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) a = max(a, __float_as_uint(x[i]) & 0x7fffffffu);
    const int field = (int)(quad_max_u32(a) >> 23);
    const int code = min(max(field - 2, 1), 254);
    uint32_t bytes = 0u;
#pragma unroll
    for (int i = 0; i < 8; i++) bytes |= nibble(x[i], code) << (4 * i);
    if (!in || slot < 0 || slot >= (int64_t)p.num_pages * p.page) return;  // per token
    const int lg = p.page == 64 ? 6 : 7;                                   // pages of 64 or 128
    const int64_t pg = slot >> lg, tok = slot & (p.page - 1);
    uint8_t* dst = p.k + pg * p.kp_s + tok * 64 + 4 * j;
    if (p.k_aligned4) {
        *reinterpret_cast<uint32_t*>(dst) = bytes;
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) dst[i] = (uint8_t)(bytes >> (8 * i));
    }
    if ((j & 3) == 0) p.ks[pg * p.ksp_s + tok * 4 + (j >> 2)] = (uint8_t)code;
}

}  // namespace

hipError_t launch_quantize_store(const QuantParams& p, hipStream_t stream) {
    if (p.N <= 0) return hipSuccess;
    QuantParams q = p;
    q.k_aligned4 = ((uintptr_t)p.k % 4 == 0 && p.kp_s % 4 == 0) ? 1 : 0;
    q.keys_aligned16 = ((uintptr_t)p.keys % 16 == 0 && p.key_rs % 8 == 0) ? 1 : 0;
    // 16 tokens a workgroup (four waves of four)
    hipLaunchKernelGGL(k_quantize_store, dim3((unsigned)((p.N + 15) / 16)), dim3(256), 0, stream, q);
    return hipGetLastError();
}

}  // namespace fp4idx
