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
// One wave per token: lane l holds elements 2l and 2l+1 (one 32-bit load of two bf16),
// so the 16 lanes of a DPP row hold exactly one 32-value block and the block maximum is
// a row reduction.  Each lane writes the byte of its two nibbles (a wave writes the
// token's 64 bytes in one coalesced store); lane 16g writes block g's code.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

// Maximum over the 16 lanes of each row (values are non-negative float bit patterns,
// whose unsigned order is their numeric order).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));   // lane ^ 1
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));   // lane ^ 2
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));  // 7 - lane%8
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));  // 15 - lane%16
    return v;
}

// Magnitude m >= 0 (already divided by the block scale) -> index of the nearest level,
// ties to the even index; above 6 -> 6.  The boundaries are the midpoints between
// levels; at a midpoint the comparison picks the even neighbour.
__device__ __forceinline__ uint32_t e2m1_index_rne(float m) {
    if (!(m > 0.25f)) return 0u;   // 0.25 ties to 0 (NaN also lands here)
    if (m < 0.75f) return 1u;      // 0.5
    if (m <= 1.25f) return 2u;     // 1.0 (0.75 and 1.25 tie to it)
    if (m < 1.75f) return 3u;      // 1.5
    if (m <= 2.5f) return 4u;      // 2.0 (1.75 and 2.5 tie to it)
    if (m < 3.5f) return 5u;       // 3.0
    if (m <= 5.0f) return 6u;      // 4.0 (3.5 and 5 tie to it)
    return 7u;                     // 6.0
}

__device__ __forceinline__ uint32_t nibble(float x, int code) {
    const float q = __builtin_ldexpf(x, 127 - code);  // exact: a power-of-two scale
    return e2m1_index_rne(__builtin_fabsf(q)) | ((__float_as_uint(x) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void k_quantize_store(const QuantParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = blockIdx.x * 4 + wave;
    if (n >= p.N) return;
    const int64_t slot = p.slots[n];
    if (slot < 0 || slot >= (int64_t)p.num_pages * p.page) return;  // uniform per wave
    const int64_t pg = slot / p.page, tok = slot - pg * p.page;
    const uint32_t two = *reinterpret_cast<const uint32_t*>(p.keys + (int64_t)n * p.key_rs + 2 * lane);
    const float x0 = __uint_as_float(two << 16), x1 = __uint_as_float(two & 0xffff0000u);
    const uint32_t a = max(__float_as_uint(x0) & 0x7fffffffu, __float_as_uint(x1) & 0x7fffffffu);
    const int field = (int)(row_max_u32(a) >> 23);
    const int code = min(max(field - 2, 1), 254);
    const uint32_t byte = nibble(x0, code) | (nibble(x1, code) << 4);
    p.k[pg * p.kp_s + tok * 64 + lane] = (uint8_t)byte;
    if ((lane & 15) == 0) p.ks[pg * p.ksp_s + tok * 4 + (lane >> 4)] = (uint8_t)code;
}

}  // namespace

hipError_t launch_quantize_store(const QuantParams& p, hipStream_t stream) {
    if (p.N <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize_store, dim3((unsigned)((p.N + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp4idx
