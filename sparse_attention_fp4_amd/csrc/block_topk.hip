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
// Each lane keeps its KMAX best (key, block) pairs sorted in registers (an insertion
// network; a step that would change no lane's list is skipped).  Strict comparison
// keeps the earlier block ahead among equal keys, so the list's first k entries are
// exactly the chosen blocks; a sorting network puts them in block order for the
// output.  Every score is read once.
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

template <int KMAX>
__global__ __launch_bounds__(256) void k_block_topk(const BlockTopkParams p) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    const int hq = blockIdx.y;
    const bool active = q < p.Tq;
    const float* col = p.scores + (int64_t)hq * p.Kt * p.Tq + (active ? q : 0);
    const int64_t step = p.Tq;

    uint32_t lk[KMAX];
    int lb[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; i++) lk[i] = 0u, lb[i] = -1;
    // block rows are read kB at a time, the next kB in flight while these are inserted
    constexpr int kB = 8;
    auto load = [&](int kb0, float (&v)[kB]) {
#pragma unroll
        for (int u = 0; u < kB; u++) {
            const int kb = kb0 + u;
            v[u] = kb < p.Kt ? col[(int64_t)kb * step] : -__builtin_inff();
        }
    };
    auto insert = [&](int kb0, const float (&v)[kB]) {
#pragma unroll
        for (int u = 0; u < kB; u++) {
            const int kb = kb0 + u;
            const uint32_t key = active ? bkey(v[u]) : 0u;  // past Kt: -inf, key 0
            if (__ballot(key > lk[KMAX - 1]) == 0ull) continue;
            // insert at the first slot holding a smaller key and shift the rest down
            // one (the list is sorted, so c[i] is false up to that slot and true after
            // it; equal keys stay in block order)
            bool c[KMAX];
#pragma unroll
            for (int i = 0; i < KMAX; i++) c[i] = key > lk[i];
#pragma unroll
            for (int i = KMAX - 1; i > 0; i--) {
                lk[i] = c[i] ? (c[i - 1] ? lk[i - 1] : key) : lk[i];
                lb[i] = c[i] ? (c[i - 1] ? lb[i - 1] : kb) : lb[i];
            }
            lk[0] = c[0] ? key : lk[0];
            lb[0] = c[0] ? kb : lb[0];
        }
    };
    float va[kB], vb[kB];
    load(0, va);
    for (int kb0 = 0; kb0 < p.Kt; kb0 += 2 * kB) {
        load(kb0 + kB, vb);
        insert(kb0, va);
        if (kb0 + kB >= p.Kt) break;
        load(kb0 + 2 * kB, va);
        insert(kb0 + kB, vb);
    }
    if (!active) return;
    // The list's first k entries are the chosen blocks: put them in block order (a
    // sorting network on the block indices; entries past k or empty sort last).
    int m = 0;
#pragma unroll
    for (int i = 0; i < KMAX; i++) {
        const bool use = i < p.k && lk[i] != 0u;
        m += use ? 1 : 0;
        lb[i] = use ? lb[i] : INT32_MAX;
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
