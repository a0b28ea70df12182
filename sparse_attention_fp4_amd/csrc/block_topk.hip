// block_topk.hip -- top-k 128-token blocks of every (head, query) from the block
// scores, gfx950.
//
// ("M3 FP4 Indexer" README, public API: the block-score interface returns scores
// without TopK; a caller takes TopK along the Ktiles dimension.)  Same rule as the
// token top-k: the k largest finite scores (-inf and NaN never chosen, -0 equal to
// +0, ties to the smaller block), listed in increasing block order, -1 padded; the
// number chosen goes to a per-(head, query) count, the metadata a block-sparse
// consumer reads next to the list.
//
// One lane per (head, query): a wave holds 64 consecutive queries of one head, so each
// step reads 64 consecutive floats of one block row of [Hq][Ktiles][Tq] (coalesced).
// A score and its block travel as one 64-bit key, (order-preserving score bits << 32)
// | ~block, so that a larger key is a larger score or an equal score of an earlier
// block.  Each lane keeps its KMAX largest keys sorted in registers: the blocks arrive
// CH at a time (the next CH in flight), a bitonic network sorts them, the elementwise
// maximum of the list and the reversed chunk holds the KMAX largest of both as a
// bitonic sequence, and a bitonic merge sorts it again -- about 40 VALU operations per
// score for KMAX = 16, against about 80 for inserting scores one at a time.  The list's
// first k entries are the chosen blocks; a sorting network puts them in block order
// for the output.  Every score is read once.
#include "device_common.hpp"
#include "fp4idx_internal.hpp"

namespace fp4idx {

namespace {

__device__ __forceinline__ uint32_t bkey(float v) {
    if (!(v > -__builtin_inff())) return 0u;  // -inf, NaN: never chosen
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// descending compare-exchange: a keeps the larger key
__device__ __forceinline__ void cx(uint64_t& a, uint64_t& b) {
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}

// Sort n keys descending (bitonic network; n a power of two).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&v)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < N; i++) {
                const int j = i ^ stride;
                if (j > i) {
                    if ((i & size) == 0) cx(v[i], v[j]);  // this run descending
                    else cx(v[j], v[i]);                  // this one ascending
                }
            }
}

// A bitonic sequence of n keys -> sorted descending.
template <int N>
__device__ __forceinline__ void merge_desc(uint64_t (&v)[N]) {
#pragma unroll
    for (int stride = N >> 1; stride > 0; stride >>= 1)
#pragma unroll
        for (int i = 0; i < N; i++)
            if ((i & stride) == 0) cx(v[i], v[i + stride]);
}

template <int KMAX>
__global__ __launch_bounds__(256) void k_block_topk(const BlockTopkParams p) {
    constexpr int CH = KMAX < 16 ? KMAX : 16;  // blocks per chunk
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int hq = blockIdx.y;
    const bool active = q < p.Tq;
    const float* col = p.scores + (int64_t)hq * p.Kt * p.Tq + (active ? q : 0);
    const int64_t step = p.Tq;

    uint64_t L[KMAX];  // the list, descending; key 0 = empty
#pragma unroll
    for (int i = 0; i < KMAX; i++) L[i] = 0ull;
    auto load = [&](int kb0, float (&v)[CH]) {
#pragma unroll
        for (int u = 0; u < CH; u++) {
            const int kb = kb0 + u;
            v[u] = kb < p.Kt ? col[(int64_t)kb * step] : -__builtin_inff();
        }
    };
    auto add_chunk = [&](int kb0, const float (&v)[CH]) {
        uint64_t c[CH];
#pragma unroll
        for (int u = 0; u < CH; u++) {
            const uint32_t key = active ? bkey(v[u]) : 0u;  // past Kt: -inf, key 0
            c[u] = key ? ((uint64_t)key << 32) | (uint32_t)~(uint32_t)(kb0 + u) : 0ull;
        }
        sort_desc<CH>(c);
        // the KMAX largest of list and chunk: L[i] against the chunk reversed (padded
        // with empty keys), a bitonic sequence
#pragma unroll
        for (int i = KMAX - CH; i < KMAX; i++) {
            const uint64_t b = c[KMAX - 1 - i];
            L[i] = L[i] > b ? L[i] : b;
        }
        merge_desc<KMAX>(L);
    };
    float va[CH], vb[CH];
    load(0, va);
    for (int kb0 = 0; kb0 < p.Kt; kb0 += 2 * CH) {
        load(kb0 + CH, vb);
        add_chunk(kb0, va);
        if (kb0 + CH >= p.Kt) break;
        load(kb0 + 2 * CH, va);
        add_chunk(kb0 + CH, vb);
    }
    if (!active) return;
    // The list's first k entries are the chosen blocks: put them in block order (a
    // sorting network on the block indices; entries past k or empty sort last).
    int lb[KMAX];
    int m = 0;
#pragma unroll
    for (int i = 0; i < KMAX; i++) {
        const bool use = i < p.k && (L[i] >> 32) != 0ull;
        m += use ? 1 : 0;
        lb[i] = use ? (int)~(uint32_t)L[i] : INT32_MAX;
    }
#pragma unroll
    for (int size = 2; size <= KMAX; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < KMAX; i++) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const int a = lb[i], b = lb[j];
                    lb[i] = up ? min(a, b) : max(a, b);
                    lb[j] = up ? max(a, b) : min(a, b);
                }
            }
    int32_t* out = p.out_idx + ((int64_t)hq * p.Tq + q) * p.k;
#pragma unroll
    for (int i = 0; i < KMAX; i++)
        if (i < p.k) out[i] = i < m ? lb[i] : -1;
    if (p.out_count) p.out_count[(int64_t)hq * p.Tq + q] = m;
}

template <int KMAX>
hipError_t launch_kmax(const BlockTopkParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((p.Tq + 255) / 256), (unsigned)p.Hq);
    hipLaunchKernelGGL(k_block_topk<KMAX>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_topk(const BlockTopkParams& p, hipStream_t stream) {
    if (p.Tq == 0) return hipSuccess;
    if (p.k <= 8) return launch_kmax<8>(p, stream);
    if (p.k <= 16) return launch_kmax<16>(p, stream);
    if (p.k <= 32) return launch_kmax<32>(p, stream);
    return launch_kmax<64>(p, stream);
}

}  // namespace fp4idx
