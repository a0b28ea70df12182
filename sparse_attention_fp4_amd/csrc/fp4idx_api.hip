// fp4idx_api.hip -- the extern "C" entry points declared in include/fp4idx.h.
//
// Each entry point checks its scalar arguments and pointer values on the host (device
// metadata is never read here), fills a parameter block and enqueues the kernels on
// the caller's stream.  Nothing is allocated and no state is kept between calls.
#include "fp4idx.h"
#include "fp4idx_internal.hpp"

#include <mutex>

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? FP4IDX_OK : FP4IDX_EHIP; }

}  // namespace

extern "C" {

int fp4idx_version(void) { return 100; }

const char* fp4idx_strerror(int code) {
    switch (code) {
        case FP4IDX_OK: return "ok";
        case FP4IDX_EINVAL: return "invalid argument";
        case FP4IDX_EUNSUPPORTED: return "unsupported size or layout";
        case FP4IDX_EALIGN: return "pointer or stride not 16-byte aligned";
        case FP4IDX_EHIP: return "HIP launch error";
        case FP4IDX_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

namespace {

// Argument checks and parameter block shared by the logits and the fused top-k entry
// points (out / out_row_stride are not checked when `need_out` is false).
int logits_params(int fmt, const uint8_t* q_fp4, int64_t q_row_stride, const uint8_t* q_scale,
                  int64_t qs_row_stride, const float* w, int64_t w_row_stride,
                  const uint8_t* k_fp4, int64_t k_page_stride, const uint8_t* k_scale,
                  int64_t ks_page_stride, const int32_t* block_table, int64_t bt_row_stride,
                  const int32_t* cu_seqlens_q, const int32_t* row_lens, int T, int B, int H,
                  int Hkv, int page_size, int num_pages, int table_width, int out_cols,
                  float* logits, int64_t out_row_stride, bool need_out, fp4idx::LogitsParams& p) {
    if (fmt != FP4IDX_MXFP4 && fmt != FP4IDX_NVFP4) return FP4IDX_EINVAL;
    if (T < 0 || B < 1 || H < 1 || Hkv < 1 || num_pages < 0 || table_width < 0 || out_cols < 0)
        return FP4IDX_EINVAL;
    if (H % Hkv != 0) return FP4IDX_EINVAL;
    if (H > 128) return FP4IDX_EUNSUPPORTED;
    if (page_size != 64 && page_size != 128) return FP4IDX_EUNSUPPORTED;
    if (T == 0 || out_cols == 0) return -1;  // nothing to do
    if (!q_fp4 || !q_scale || !w || !cu_seqlens_q || !row_lens || (need_out && !logits))
        return FP4IDX_EINVAL;
    if (num_pages > 0 && table_width > 0 && (!k_fp4 || !k_scale || !block_table))
        return FP4IDX_EINVAL;
    const int G = fmt == FP4IDX_MXFP4 ? 4 : 8;
    if (q_row_stride < (int64_t)H * 64 || qs_row_stride < (int64_t)H * G || w_row_stride < H ||
        (need_out && out_row_stride < out_cols) || bt_row_stride < table_width)
        return FP4IDX_EINVAL;
    // output rows of one row block are addressed with 32-bit offsets
    if (need_out && out_row_stride > ((int64_t)1 << 27)) return FP4IDX_EUNSUPPORTED;
    if (k_page_stride < (int64_t)Hkv * page_size * 64 || ks_page_stride < (int64_t)Hkv * page_size * G)
        return FP4IDX_EINVAL;
    if (!aligned16(q_fp4) || (q_row_stride & 15) || !aligned16(k_fp4) || (k_page_stride & 15))
        return FP4IDX_EALIGN;
    if (num_pages > 0 && table_width > 0 && (!aligned16(k_scale) || (ks_page_stride & 15)))
        return FP4IDX_EALIGN;
    p = fp4idx::LogitsParams{};
    p.q = q_fp4;
    p.q_rs = q_row_stride;
    p.qs = q_scale;
    p.qs_rs = qs_row_stride;
    p.w = w;
    p.w_rs = w_row_stride;
    p.k = k_fp4;
    p.kp_s = k_page_stride;
    p.ks = k_scale;
    p.ksp_s = ks_page_stride;
    p.bt = block_table;
    p.bt_rs = bt_row_stride;
    p.cu = cu_seqlens_q;
    p.lens = row_lens;
    p.out = logits;
    p.out_rs = out_row_stride;
    p.T = T;
    p.B = B;
    p.H = H;
    p.Hkv = Hkv;
    p.page = page_size;
    p.num_pages = (k_fp4 && block_table) ? num_pages : 0;
    p.W = table_width;
    p.out_cols = out_cols;
    p.fmt = fmt;
    p.G = G;
    p.R = H / Hkv;
    return FP4IDX_OK;
}

}  // namespace

int fp4idx_logits_paged(int fmt,
                        const uint8_t* q_fp4, int64_t q_row_stride,
                        const uint8_t* q_scale, int64_t qs_row_stride,
                        const float* w, int64_t w_row_stride,
                        const uint8_t* k_fp4, int64_t k_page_stride,
                        const uint8_t* k_scale, int64_t ks_page_stride,
                        const int32_t* block_table, int64_t bt_row_stride,
                        const int32_t* cu_seqlens_q, const int32_t* row_lens,
                        int T, int B, int H, int Hkv, int page_size, int num_pages,
                        int table_width, int out_cols,
                        float* logits, int64_t out_row_stride,
                        void* stream) {
    fp4idx::LogitsParams p;
    const int rc = logits_params(fmt, q_fp4, q_row_stride, q_scale, qs_row_stride, w, w_row_stride,
                                 k_fp4, k_page_stride, k_scale, ks_page_stride, block_table,
                                 bt_row_stride, cu_seqlens_q, row_lens, T, B, H, Hkv, page_size,
                                 num_pages, table_width, out_cols, logits, out_row_stride, true, p);
    if (rc != FP4IDX_OK) return rc < 0 ? FP4IDX_OK : rc;
    return hip_status(fp4idx::launch_logits(p, (hipStream_t)stream));
}

size_t fp4idx_logits_topk_workspace_bytes(int fmt, int T, int B, int H, int Hkv, int page_size,
                                          int table_width, int out_cols, int k) {
    if ((fmt != FP4IDX_MXFP4 && fmt != FP4IDX_NVFP4) || T <= 0 || B < 1 || H < 1 || Hkv < 1 ||
        H % Hkv != 0 || H > 128 || (page_size != 64 && page_size != 128) || table_width < 0 ||
        out_cols <= 0 || k < 1)
        return 0;
    fp4idx::LogitsParams p{};
    p.T = T;
    p.B = B;
    p.H = H;
    p.Hkv = Hkv;
    p.page = page_size;
    p.W = table_width;
    p.out_cols = out_cols;
    p.fmt = fmt;
    p.G = fmt == FP4IDX_MXFP4 ? 4 : 8;
    p.R = H / Hkv;
    return fp4idx::logits_topk_workspace_bytes(p, k);
}

namespace {

// Checks shared by the fused entry point and its allocation-free variant.  Returns
// FP4IDX_OK with `p` filled when there is work, -1 when the call is complete (no rows,
// or nothing to select: the output padding is then enqueued), else an error code.
int logits_topk_prepare(int fmt, const uint8_t* q_fp4, int64_t q_row_stride,
                        const uint8_t* q_scale, int64_t qs_row_stride, const float* w,
                        int64_t w_row_stride, const uint8_t* k_fp4, int64_t k_page_stride,
                        const uint8_t* k_scale, int64_t ks_page_stride,
                        const int32_t* block_table, int64_t bt_row_stride,
                        const int32_t* cu_seqlens_q, const int32_t* row_lens, int T, int B,
                        int H, int Hkv, int page_size, int num_pages, int table_width,
                        int out_cols, int k, int32_t* out_idx, float* out_vals, void* stream,
                        fp4idx::LogitsParams& p, size_t& need) {
    if (k < 1) return FP4IDX_EINVAL;
    if (k > 2048 || out_cols > (1 << 24)) return FP4IDX_EUNSUPPORTED;
    const int rc = logits_params(fmt, q_fp4, q_row_stride, q_scale, qs_row_stride, w, w_row_stride,
                                 k_fp4, k_page_stride, k_scale, ks_page_stride, block_table,
                                 bt_row_stride, cu_seqlens_q, row_lens, T, B, H, Hkv, page_size,
                                 num_pages, table_width, out_cols, nullptr, 0, false, p);
    if (rc > 0) return rc;
    if (!out_idx && T > 0) return FP4IDX_EINVAL;
    if (rc < 0) {  // no rows or no columns: nothing is selected
        if (T == 0) return -1;
        const int e = hip_status(fp4idx::launch_fill_empty_topk(T, k, out_idx, out_vals, (hipStream_t)stream));
        return e == FP4IDX_OK ? -1 : e;
    }
    need = fp4idx::logits_topk_workspace_bytes(p, k);
    if (need == 0) return FP4IDX_EUNSUPPORTED;
    return FP4IDX_OK;
}

// ---- scratch of the allocation-free entry point: one array per GPU, in the code
// object, found once per device; host code uses only the looked-up device address.
constexpr size_t kNoAllocScratchBytes = FP4IDX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4IDX_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP4IDX_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FP4IDX_OK;
}

}  // namespace

int fp4idx_logits_topk_paged(int fmt,
                             const uint8_t* q_fp4, int64_t q_row_stride,
                             const uint8_t* q_scale, int64_t qs_row_stride,
                             const float* w, int64_t w_row_stride,
                             const uint8_t* k_fp4, int64_t k_page_stride,
                             const uint8_t* k_scale, int64_t ks_page_stride,
                             const int32_t* block_table, int64_t bt_row_stride,
                             const int32_t* cu_seqlens_q, const int32_t* row_lens,
                             int T, int B, int H, int Hkv, int page_size, int num_pages,
                             int table_width, int out_cols, int k,
                             int32_t* out_idx, float* out_vals,
                             void* workspace, size_t workspace_bytes, void* stream) {
    fp4idx::LogitsParams p;
    size_t need = 0;
    const int rc = logits_topk_prepare(fmt, q_fp4, q_row_stride, q_scale, qs_row_stride, w,
                                       w_row_stride, k_fp4, k_page_stride, k_scale, ks_page_stride,
                                       block_table, bt_row_stride, cu_seqlens_q, row_lens, T, B, H,
                                       Hkv, page_size, num_pages, table_width, out_cols, k, out_idx,
                                       out_vals, stream, p, need);
    if (rc != FP4IDX_OK) return rc < 0 ? FP4IDX_OK : rc;
    if (!workspace || workspace_bytes < need || !aligned256(workspace)) return FP4IDX_EWORKSPACE;
    return hip_status(fp4idx::launch_logits_topk(p, k, out_idx, out_vals, workspace,
                                                 workspace_bytes, (hipStream_t)stream));
}

int fp4idx_logits_topk_paged_noalloc(int fmt,
                                     const uint8_t* q_fp4, int64_t q_row_stride,
                                     const uint8_t* q_scale, int64_t qs_row_stride,
                                     const float* w, int64_t w_row_stride,
                                     const uint8_t* k_fp4, int64_t k_page_stride,
                                     const uint8_t* k_scale, int64_t ks_page_stride,
                                     const int32_t* block_table, int64_t bt_row_stride,
                                     const int32_t* cu_seqlens_q, const int32_t* row_lens,
                                     int T, int B, int H, int Hkv, int page_size, int num_pages,
                                     int table_width, int out_cols, int k,
                                     int32_t* out_idx, float* out_vals, void* stream) {
    fp4idx::LogitsParams p;
    size_t need = 0;
    const int rc = logits_topk_prepare(fmt, q_fp4, q_row_stride, q_scale, qs_row_stride, w,
                                       w_row_stride, k_fp4, k_page_stride, k_scale, ks_page_stride,
                                       block_table, bt_row_stride, cu_seqlens_q, row_lens, T, B, H,
                                       Hkv, page_size, num_pages, table_width, out_cols, k, out_idx,
                                       out_vals, stream, p, need);
    if (rc != FP4IDX_OK) return rc < 0 ? FP4IDX_OK : rc;
    if (need > kNoAllocScratchBytes) return FP4IDX_EWORKSPACE;
    void* ws = nullptr;
    const int src = scratch_of_current_device(&ws);
    if (src != FP4IDX_OK) return src;
    return hip_status(fp4idx::launch_logits_topk(p, k, out_idx, out_vals, ws, kNoAllocScratchBytes,
                                                 (hipStream_t)stream));
}

int fp4idx_block_scores(int fmt,
                        const uint8_t* q_fp4, const uint8_t* q_scale,
                        const uint8_t* k_fp4, const uint8_t* k_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* cu_page_offsets, const int32_t* kv_indices,
                        const int32_t* qo_offset,
                        int B, int Tq, int Hq, int Hkv, int num_pages,
                        int max_seqlen_q, int max_seqlen_k, int causal,
                        float* scores, void* stream) {
    if (fmt != FP4IDX_MXFP4 && fmt != FP4IDX_NVFP4) return FP4IDX_EINVAL;
    if (max_seqlen_q <= 0) return FP4IDX_EINVAL;
    if (B < 1 || Tq < 0 || Hq < 1 || Hkv < 1 || num_pages < 0 || max_seqlen_k < 0)
        return FP4IDX_EINVAL;
    if (Hq % Hkv != 0) return FP4IDX_EINVAL;
    if (qo_offset && !causal) return FP4IDX_EINVAL;
    if (Tq == 0 || max_seqlen_k == 0) return FP4IDX_OK;
    if (!q_fp4 || !q_scale || !cu_seqlens_q || !cu_seqlens_k || !cu_page_offsets || !scores)
        return FP4IDX_EINVAL;
    if (num_pages > 0 && (!k_fp4 || !k_scale || !kv_indices)) return FP4IDX_EINVAL;
    if (!aligned16(q_fp4) || (k_fp4 && !aligned16(k_fp4)) || (k_scale && !aligned16(k_scale)))
        return FP4IDX_EALIGN;
    fp4idx::BlockParams p{};
    p.q = q_fp4;
    p.qs = q_scale;
    p.k = k_fp4;
    p.ks = k_scale;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.cu_p = cu_page_offsets;
    p.kv_indices = kv_indices;
    p.qo_offset = qo_offset;
    p.scores = scores;
    p.B = B;
    p.Tq = Tq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.num_pages = (k_fp4 && kv_indices) ? num_pages : 0;
    p.max_seqlen_q = max_seqlen_q;
    p.max_seqlen_k = max_seqlen_k;
    p.causal = causal ? 1 : 0;
    p.fmt = fmt;
    p.G = fmt == FP4IDX_MXFP4 ? 4 : 8;
    p.R = Hq / Hkv;
    p.ktiles = (max_seqlen_k + 127) / 128;
    return hip_status(fp4idx::launch_block_scores(p, (hipStream_t)stream));
}

int fp4idx_quantize_store_k(const uint16_t* keys, int64_t key_row_stride, const int64_t* slots, int N,
                            uint8_t* k_fp4, int64_t k_page_stride, uint8_t* k_scale,
                            int64_t ks_page_stride, int page_size, int num_pages, void* stream) {
    if (N < 0 || num_pages < 0) return FP4IDX_EINVAL;
    if (page_size != 64 && page_size != 128) return FP4IDX_EUNSUPPORTED;
    if (N == 0 || num_pages == 0) return FP4IDX_OK;
    if (!keys || !slots || !k_fp4 || !k_scale) return FP4IDX_EINVAL;
    if (key_row_stride < 128 || k_page_stride < (int64_t)page_size * 64 ||
        ks_page_stride < (int64_t)page_size * 4)
        return FP4IDX_EINVAL;
    if (((uintptr_t)keys & 3u) || (key_row_stride & 1)) return FP4IDX_EALIGN;
    fp4idx::QuantParams p{};
    p.keys = keys;
    p.key_rs = key_row_stride;
    p.slots = slots;
    p.k = k_fp4;
    p.kp_s = k_page_stride;
    p.ks = k_scale;
    p.ksp_s = ks_page_stride;
    p.N = N;
    p.page = page_size;
    p.num_pages = num_pages;
    return hip_status(fp4idx::launch_quantize_store(p, (hipStream_t)stream));
}

int fp4idx_block_topk(const float* scores, int Hq, int Ktiles, int Tq, int k,
                      int32_t* out_idx, int32_t* out_count, void* stream) {
    if (Hq < 1 || Ktiles < 0 || Tq < 0 || k < 1) return FP4IDX_EINVAL;
    if (k > 64) return FP4IDX_EUNSUPPORTED;
    if (Tq == 0) return FP4IDX_OK;
    if (!out_idx || (Ktiles > 0 && !scores)) return FP4IDX_EINVAL;
    if ((int64_t)Hq * Ktiles * Tq > ((int64_t)1 << 40)) return FP4IDX_EUNSUPPORTED;
    fp4idx::BlockTopkParams p{};
    p.scores = scores;
    p.Hq = Hq;
    p.Kt = Ktiles;
    p.Tq = Tq;
    p.k = k;
    p.out_idx = out_idx;
    p.out_count = out_count;
    return hip_status(fp4idx::launch_block_topk(p, (hipStream_t)stream));
}

namespace {

// bit length of page_size - 1, at least 1 (slot layout of the sparse attention)
int qsa_offset_bits(int page_size) {
    int b = 1;
    while (b < 31 && ((int64_t)1 << b) < (int64_t)page_size) b++;
    return b;
}

bool qsa_slot_fits(int num_cache_blocks, int ob) {
    return ((int64_t)num_cache_blocks << ob) < ((int64_t)1 << 31);
}

}  // namespace

int fp4idx_qsa_slots(const int32_t* indices, int64_t indices_row_stride, int rows, int topk,
                     const int32_t* block_table, int64_t block_table_row_stride,
                     int num_requests, int table_width, const int32_t* token_to_req,
                     int num_cache_blocks, int page_size,
                     int32_t* slots, int64_t slots_row_stride, int slot_cols, void* stream) {
    if (rows < 0 || topk < 1 || slot_cols < topk || page_size < 1 || num_requests < 1 ||
        table_width < 1 || num_cache_blocks < 1)
        return FP4IDX_EINVAL;
    if (indices_row_stride < topk || block_table_row_stride < table_width ||
        slots_row_stride < slot_cols)
        return FP4IDX_EINVAL;
    const int ob = qsa_offset_bits(page_size);
    if (!qsa_slot_fits(num_cache_blocks, ob)) return FP4IDX_EINVAL;
    if (rows == 0) return FP4IDX_OK;
    if (!indices || !block_table || !token_to_req || !slots) return FP4IDX_EINVAL;
    if ((int64_t)rows * ((slot_cols + 255) / 256) > 0x7fffffff) return FP4IDX_EUNSUPPORTED;
    fp4idx::QsaSlotParams p{};
    p.ind = indices;
    p.ind_rs = indices_row_stride;
    p.rows = rows;
    p.topk = topk;
    p.bt = block_table;
    p.bt_rs = block_table_row_stride;
    p.num_req = num_requests;
    p.width = table_width;
    p.t2r = token_to_req;
    p.num_blocks = num_cache_blocks;
    p.page = page_size;
    p.ob = ob;
    p.slots = slots;
    p.slots_rs = slots_row_stride;
    p.slot_cols = slot_cols;
    return hip_status(fp4idx::launch_qsa_slots(p, (hipStream_t)stream));
}

int fp4idx_qsa_decode(const uint16_t* q, int64_t q_row_stride, int64_t q_head_stride,
                      const uint8_t* k_cache, const uint8_t* v_cache,
                      int64_t block_stride, int64_t token_stride,
                      int64_t k_head_stride, int64_t v_head_stride,
                      int num_cache_blocks, int page_size,
                      const int32_t* slots, int64_t slots_row_stride,
                      const int32_t* indices, int64_t indices_row_stride, int topk,
                      int rows, int Hq, int Hkv, int head_dim,
                      float softmax_scale, float output_scale,
                      const uint16_t* gate, int64_t gate_row_stride, int64_t gate_head_stride,
                      uint16_t* out, int64_t out_row_stride, int64_t out_head_stride,
                      void* stream) {
    if (rows < 0 || topk < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || page_size < 1 ||
        num_cache_blocks < 1)
        return FP4IDX_EINVAL;
    const int ob = qsa_offset_bits(page_size);
    if (!qsa_slot_fits(num_cache_blocks, ob)) return FP4IDX_EINVAL;
    if (head_dim != 128 || Hq / Hkv > 16) return FP4IDX_EUNSUPPORTED;
    if (block_stride < 0 || token_stride < 0 || block_stride >= ((int64_t)1 << 32) ||
        token_stride >= ((int64_t)1 << 32))
        return FP4IDX_EUNSUPPORTED;
    if (rows == 0) return FP4IDX_OK;
    if (!q || !k_cache || !v_cache || !slots || !indices || !gate || !out) return FP4IDX_EINVAL;
    if (indices_row_stride <= topk || slots_row_stride < 0) return FP4IDX_EINVAL;
    if ((int64_t)rows * Hkv > 0x7fffffff) return FP4IDX_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(gate) || !aligned16(out) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(slots))
        return FP4IDX_EALIGN;
    if ((q_row_stride | q_head_stride | gate_row_stride | gate_head_stride | out_row_stride |
         out_head_stride) & 7)
        return FP4IDX_EALIGN;
    if ((block_stride | token_stride | k_head_stride | v_head_stride) & 15) return FP4IDX_EALIGN;
    fp4idx::QsaDecodeParams p{};
    p.q = q;
    p.q_rs = q_row_stride;
    p.q_hs = q_head_stride;
    p.k = k_cache;
    p.v = v_cache;
    p.bs = block_stride;
    p.ts = token_stride;
    p.khs = k_head_stride;
    p.vhs = v_head_stride;
    p.slots = slots;
    p.slots_rs = slots_row_stride;
    p.ind = indices;
    p.ind_rs = indices_row_stride;
    p.topk = topk;
    p.rows = rows;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.ob = ob;
    p.num_blocks = num_cache_blocks;
    p.page = page_size;
    p.score_scale = (float)((double)softmax_scale * 1.4426950408889634);
    p.out_scale = output_scale;
    p.gate = gate;
    p.gate_rs = gate_row_stride;
    p.gate_hs = gate_head_stride;
    p.out = out;
    p.out_rs = out_row_stride;
    p.out_hs = out_head_stride;
    return hip_status(fp4idx::launch_qsa_decode(p, (hipStream_t)stream));
}

int fp4idx_set_topk_wait_limit(int polls) {
    return fp4idx::set_topk_wait_limit(polls);
}

size_t fp4idx_topk_workspace_bytes(int rows, int cols, int k) {
    if (rows <= 0 || cols <= 0 || k <= 0) return 0;
    return fp4idx::topk_workspace_bytes(rows, cols, k);
}

int fp4idx_topk(const float* scores, int64_t row_stride, int rows, int cols,
                const int32_t* row_lens, int k,
                int32_t* out_idx, float* out_vals,
                void* workspace, size_t workspace_bytes, void* stream) {
    if (rows < 0 || cols < 0 || k < 1) return FP4IDX_EINVAL;
    if (k > 8192 || cols > (1 << 19)) return FP4IDX_EUNSUPPORTED;
    if (rows == 0) return FP4IDX_OK;
    if (!out_idx) return FP4IDX_EINVAL;
    if (cols > 0 && (!scores || row_stride < cols)) return FP4IDX_EINVAL;
    size_t need = fp4idx_topk_workspace_bytes(rows, cols, k);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned256(workspace)))
        return FP4IDX_EWORKSPACE;
    fp4idx::TopkParams p{};
    p.scores = scores;
    p.row_stride = row_stride;
    p.rows = rows;
    p.cols = cols;
    p.k = k;
    p.row_lens = row_lens;
    p.out_idx = out_idx;
    p.out_vals = out_vals;
    p.workspace = need > 0 ? workspace : nullptr;
    return hip_status(fp4idx::launch_topk(p, (hipStream_t)stream));
}

}  // extern "C"
