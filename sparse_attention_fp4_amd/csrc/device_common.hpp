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
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
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

// Request that owns row t of a prefix-sum table cu[0..B] (cu[0] == 0, nondecreasing):
// the largest b with cu[b] <= t.  The whole wave scans 64 entries per load and counts
// the prefix with a ballot, so the usual B <= 64 case costs one load.  t must be
// wave-uniform.  `end` = cu[b+1]; ok = false when t >= cu[B] (no request owns t).
struct RowRequest {
    int b;
    int end;
    bool ok;
};

__device__ __forceinline__ RowRequest find_request(const int32_t* __restrict__ cu, int B, int t) {
    const int lane = threadIdx.x & 63;
    int m = 0;  // number of entries of cu[0..B] that are <= t (a prefix)
    int end = 0x7fffffff;
    for (int base = 0; base <= B; base += 64) {
        const int idx = base + lane;
        const int v = idx <= B ? cu[idx] : 0x7fffffff;
        const unsigned long long le = __ballot(v <= t);
        const int cnt = __popcll(le);
        m += cnt;
        if (cnt < 64) {
            end = __shfl(v, cnt);  // first entry > t (or past the table)
            break;
        }
    }
    RowRequest r;
    r.ok = m >= 1 && m <= B;
    r.b = r.ok ? m - 1 : (m >= 1 ? min(m - 1, B - 1) : 0);
    r.end = __builtin_amdgcn_readfirstlane(end);
    r.b = __builtin_amdgcn_readfirstlane(r.b);
    return r;
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return zeros
// without touching memory (a zero-byte descriptor makes every load return zeros).
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw-buffer descriptor, word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kRsrcWord3);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The dispatcher deals consecutive workgroups to the chip's 8 dies (XCDs, each with its
// own L2) in turn.  xcd_order maps a dispatched block index to a logical one so that runs
// of `run` consecutive logical blocks land on one die: neighbours that read the same data
// share an L2.  The grid must be a multiple of 8 * run (xcd_grid); logical indices past
// the real block count must exit.
__device__ __forceinline__ int xcd_order(int b, int run) {
    const int k = b >> 3;
    return (k / run) * (8 * run) + (b & 7) * run + k % run;
}
inline int64_t xcd_grid(int64_t blocks, int run) {
    const int64_t g = 8 * (int64_t)run;
    return (blocks + g - 1) / g * g;
}

// Workgroup barrier that orders LDS only.  Every barrier in this library guards data in
// LDS; __syncthreads() would also wait for each wave's outstanding global loads and
// stores, which keeps prefetched data from staying in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// v[l] + v[l ^ 32] and v[l] + v[l ^ 16] with the gfx950 lane-swap instructions (plain
// VALU operations, no LDS round trip).  Called with the same value in both operands,
// v_permlane32_swap returns (v[l & 31], v[l | 32]) and v_permlane16_swap returns the
// matching pair for 16-lane rows, so the two halves hold both addends.
__device__ __forceinline__ float add_lane_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_lane_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_lane_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int max_lane_xor32i(int v) {
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int max_lane_xor16i(int v) {
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float max_lane_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ v4i load16(const uint8_t* p) {
    return *reinterpret_cast<const v4i*>(p);
}

// NVFP4 E4M3 scale code -> (power-of-two factor 2^a as fp32, integer factor b) with
// value = 2^a * b exactly: a normal code (exponent field e > 0, mantissa m) is
// 2^(e-10) * (8 + m); a subnormal code is 2^-9 * m.  The sign goes into b.
// NaN codes (0x7F, 0xFF) give a NaN integer factor, so every value they scale (zeros
// included) decodes to NaN.
__device__ __forceinline__ void e4m3_split(uint32_t code, float& pow2, float& b) {
    uint32_t e = (code >> 3) & 15u, m = code & 7u;
    int a = e ? (int)e - 10 : -9;
    float mag = e ? (float)(8u + m) : (float)m;
    b = (code & 0x80u) ? -mag : mag;
    // 2^a built in the exponent field (a in [-10, 5])
    pow2 = __uint_as_float((uint32_t)(a + 127) << 23);
    if ((code & 0x7Fu) == 0x7Fu) b = __builtin_nanf("");
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

// Reduction over the 64 lanes of a wave without LDS: DPP quad permutations and row
// mirrors combine the 16 lanes of each row, then the two lane-swap instructions combine
// rows and halves.  Every lane receives the result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));   // lane ^ 1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));   // lane ^ 2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));  // 7 - lane%8
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));  // 15 - lane%16
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op((uint32_t)r16[0], (uint32_t)r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op((uint32_t)r32[0], (uint32_t)r32[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_sum_i32(int v) {
    return (int)wave_reduce((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS): three
// row_shr steps and two masked ones give each 16-lane row its scan, then row_bcast:15
// and row_bcast:31 carry row totals into the rows above (GCN/CDNA cross-lane scan).
__device__ __forceinline__ int wave_incl_scan(int x) {
    int v = x;
    v += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xf, 0xf, true);   // row_shr:3
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, false);  // row_shr:4, lanes 4..15
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, false);  // row_shr:8, lanes 8..15
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Exclusive prefix sum of x over the NT threads of a workgroup (wave scans, then a scan
// of the wave totals in every wave).  wtot: LDS scratch of NT/64 ints.  Ends with a
// barrier.
template <int NT>
__device__ __forceinline__ void block_excl_scan(int x, int* wtot, int& excl, int& total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = wave_incl_scan(x);
    if (lane == 63) wtot[wave] = s;
    lds_barrier();
    const int t = lane < NW ? wtot[lane] : 0;
    const int ts = wave_incl_scan(t);
    const int before = wave > 0 ? __builtin_amdgcn_readlane(ts, wave - 1) : 0;
    total = __builtin_amdgcn_readlane(ts, NW - 1);
    excl = before + s - x;
    lds_barrier();
}

// Thread-parallel bin pick: thread t owns PER bins listed in "before" order (c[b] =
// count, bin[b] = bin index).  Finds the bin that holds the kk-th element of that
// order; out[0] = bin, out[1] = elements before it, out[2] = total, out[3] = the bin's
// own count.  out[0], out[1] and out[3] are left untouched when total < kk.  Ends with
// a barrier.
template <int NT, int PER>
__device__ __forceinline__ void pick_bin(const int (&c)[PER], const int (&bin)[PER], int kk, int* wtot,
                                         int* out) {
    int s = 0;
#pragma unroll
    for (int b = 0; b < PER; b++) s += c[b];
    int excl, total;
    block_excl_scan<NT>(s, wtot, excl, total);
    if (threadIdx.x == 0) out[2] = total;
    if (excl < kk && kk <= excl + s) {
#pragma unroll
        for (int b = 0; b < PER; b++) {
            if (excl + c[b] >= kk) {
                out[0] = bin[b];
                out[1] = excl;
                out[3] = c[b];
                break;
            }
            excl += c[b];
        }
    }
    lds_barrier();
}

}  // namespace fp4idx
