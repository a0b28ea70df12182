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
//   pass 1: each lane keeps its KMAX best (key, block) pairs sorted in registers (an
//           insertion network; a step that would change no lane's list is skipped).
//           Strict comparison keeps the earlier block ahead among equal keys, so the
//           list's k-th key T and the number of list entries equal to T ("need")
//           settle the choice.
//   pass 2: the lane walks its blocks again in order and writes every block above T
//           and the first `need` blocks equal to T.
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
    float nxt = p.Kt > 0 ? col[0] : 0.f;
    for (int kb = 0; kb < p.Kt; kb++) {
        const float v = nxt;
        if (kb + 1 < p.Kt) nxt = col[(kb + 1) * step];
        uint32_t key = active ? bkey(v) : 0u;
        if (__ballot(key > lk[KMAX - 1]) == 0ull) continue;
        int b = kb;
#pragma unroll
        for (int i = 0; i < KMAX; i++) {
            const bool gt = key > lk[i];
            const uint32_t tk = lk[i];
            const int tb = lb[i];
            lk[i] = gt ? key : tk;
            lb[i] = gt ? b : tb;
            key = gt ? tk : key;
            b = gt ? tb : b;
        }
    }
    if (!active) return;
    // T = the k-th key (0: fewer than k valid blocks, all of them are chosen)
    uint32_t T = 0u;
#pragma unroll
    for (int i = 0; i < KMAX; i++)
        if (i == p.k - 1) T = lk[i];
    int need = 0;
#pragma unroll
    for (int i = 0; i < KMAX; i++)
        if (i < p.k && lk[i] == T && T != 0u) need++;

    int32_t* out = p.out_idx + ((int64_t)hq * p.Tq + q) * p.k;
    int pos = 0, seen = 0;
    for (int kb = 0; kb < p.Kt; kb++) {
        const uint32_t key = bkey(col[kb * step]);
        bool take;
        if (T == 0u) {
            take = key != 0u;
        } else {
            take = key > T || (key == T && seen < need);
            seen += key == T ? 1 : 0;
        }
        if (take) out[pos++] = kb;
    }
    for (int i = pos; i < p.k; i++) out[i] = -1;
    if (p.out_count) p.out_count[(int64_t)hq * p.Tq + q] = pos;
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
