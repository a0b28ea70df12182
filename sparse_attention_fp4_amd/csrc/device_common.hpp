// device_common.hpp -- gfx950 building blocks shared by the fp4idx kernels.
//
// Lane layouts of the two MFMA shapes used here were measured on gfx950 (a probe that
// multiplies random operands and compares with a CPU matmul under each candidate
// layout):
//   V_MFMA_SCALE_F32_16X16X128_F8F6F4 with FP4 (E2M1) operands, format code 4:
//     lane l supplies row (l % 16) of A (column (l % 16) of B) and the 32 consecutive
//     K elements [32*(l/16), 32*(l/16)+32) as 16 bytes in the low four dwords of the
//     8-dword operand, bytes in memory order; its E8M0 scale operand covers exactly those
//     32 elements (byte 0 selected by op_sel 0).
//   V_MFMA_F32_16X16X32_F16: lane l supplies row (l % 16) of A (column of B) and 8
//     consecutive K elements; any K permutation applied to both operands gives the same
//     products.
//   Both write D[4*(l/16) + i][l % 16] to element i of the lane's 4-float result.
// Rounding of the scaled FP4 MFMA, measured on 2^20 random tiles: each 32-element block
// sum is formed exactly and scaled, and the four block values are then added to C in
// block order in fp32 with round-to-nearest-even.  That model matched every tile with
// E8M0 codes in 123..131; with codes 120..134 it matched 98.8% and every result stayed
// within 2 * 2^-24 * sum|terms|.  So a dot is correctly rounded unless an intermediate
// block sum rounds (about 1e-5 of dots at codes 123..131), and is always within three
// fp32 roundings of the exact value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// D = A * B + C over one 16x16x128 FP4 tile with one E8M0 scale per 32 elements.
__device__ __forceinline__ v4f mfma_fp4_16x16x128(v4i a, int scale_a, v4i b, int scale_b, v4f c) {
    v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, scale_a, 0, scale_b);
}

// D = A * B + C over one 16x16x32 fp16 tile.
__device__ __forceinline__ v4f mfma_f16_16x16x32(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Largest b in [0, B) with cu[b] <= t (cu[0] == 0).  Wave-uniform when t is.
__device__ __forceinline__ int find_request(const int32_t* __restrict__ cu, int B, int t) {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ v4i load16(const uint8_t* p) {
    return *reinterpret_cast<const v4i*>(p);
}

// NVFP4 E4M3 scale code -> (power-of-two factor 2^a as fp32, integer factor b) with
// value = 2^a * b exactly: a normal code (exponent field e > 0, mantissa m) is
// 2^(e-10) * (8 + m); a subnormal code is 2^-9 * m.  The sign goes into b.
// NaN codes (0x7F, 0xFF) give a NaN power factor.
__device__ __forceinline__ void e4m3_split(uint32_t code, float& pow2, float& b) {
    uint32_t e = (code >> 3) & 15u, m = code & 7u;
    int a = e ? (int)e - 10 : -9;
    float mag = e ? (float)(8u + m) : (float)m;
    b = (code & 0x80u) ? -mag : mag;
    // 2^a built in the exponent field (a in [-10, 5])
    pow2 = __uint_as_float((uint32_t)(a + 127) << 23);
    if ((code & 0x7Fu) == 0x7Fu) pow2 = __builtin_nanf("");
}

// The eight E2M1 values of one dword (bytes 0..3, low nibble first) times 2^a * b, as fp16.
// The converter scales by the exponent of its fp32 scale operand only, so the integer
// factor b is applied afterwards with a packed fp16 multiply; every intermediate is an
// exact fp16 value (at most 6 significant bits, magnitude in [2^-11, 2880]).
__device__ __forceinline__ v8h decode8_f16(uint32_t packed, float pow2, float b) {
    v2h bb = {(_Float16)b, (_Float16)b};
    v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, pow2, 0) * bb;
    v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, pow2, 1) * bb;
    v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, pow2, 2) * bb;
    v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, pow2, 3) * bb;
    v8h r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return r;
}

}  // namespace fp4idx
