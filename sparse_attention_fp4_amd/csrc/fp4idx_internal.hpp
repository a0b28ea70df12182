// fp4idx_internal.hpp -- parameter blocks and launchers shared by the host entry points
// (fp4idx_api.hip) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4idx {

struct LogitsParams {
    const uint8_t* q;
    int64_t q_rs;        // bytes between query rows
    const uint8_t* qs;
    int64_t qs_rs;       // bytes between query-scale rows
    const float* w;
    int64_t w_rs;        // floats between weight rows
    const uint8_t* k;
    int64_t kp_s;        // bytes between key pages
    const uint8_t* ks;
    int64_t ksp_s;       // bytes between key-scale pages
    const int32_t* bt;
    int64_t bt_rs;       // int32 elements between block-table rows
    const int32_t* cu;   // [B+1]
    const int32_t* lens; // [T]
    float* out;
    int64_t out_rs;      // floats between logits rows
    int T, B, H, Hkv, page, num_pages, W, out_cols;
    int fmt;
    int G;               // scale groups per 128 values (4 or 8)
    int R;               // H / Hkv
    int tiles_per_kv;    // A tiles per key head
    int n_tiles;         // Hkv * tiles_per_kv
    int ppw;             // pages per wave
    int n_wchunks;       // column chunks (of ppw pages) per row block
    int n_wgchunks;      // workgroups per row block (one chunk per wave)
    int n_rowblocks;
    int rows_per_block;  // RG: query rows sharing one A tile
    // Fused scoring (top-k candidates instead of logits; `out` unused when cand is set):
    // a score >= lo[t] (and > -inf) of row t is written as (value bits | column << 32)
    // into cand[t][c0 + i], c0 = the first column of the wave's chunk and i the rank of
    // that column among the chunk's kept columns; counts[t][chunk] receives the number
    // kept.  flags (optional): only row blocks with a flagged row run, and a flagged row
    // keeps every score.
    const float* lo;
    const int32_t* flags;
    uint64_t* cand;
    int64_t cand_rs;     // entries between candidate rows
    int32_t* counts;
    int counts_rs;       // ints between count rows
    // Optional: zero_words (< 2^31) words from `zero` are cleared by the launch (a
    // region the next kernels on the stream need zeroed, cleared without a kernel of its
    // own); zero_per_block is set by the launcher.
    uint32_t* zero;
    int zero_words;
    int zero_per_block;
};

// Row blocks, tiles and column chunks of a logits launch (fills rows_per_block,
// tiles_per_kv, n_tiles, n_rowblocks, ppw, n_wchunks, n_wgchunks).  false when the
// head layout needs more A tiles than a block holds.
bool plan_logits(LogitsParams& p);

struct BlockParams {
    const uint8_t* q;
    const uint8_t* qs;
    const uint8_t* k;
    const uint8_t* ks;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* cu_p;
    const int32_t* kv_indices;
    const int32_t* qo_offset;  // nullable
    float* scores;
    int B, Tq, Hq, Hkv, num_pages, max_seqlen_q, max_seqlen_k, causal;
    int fmt, G, R;
    int ktiles;
    int q_tiles;         // query tiles of 16 tokens in the grid's y dimension
    int kb_chunk;        // 128-key blocks per wave (the key range is cut in chunks)
    int n_kchunks;       // chunks of kb_chunk blocks over Ktiles
};

struct TopkParams {
    const float* scores;
    int64_t row_stride;
    int rows, cols, k;
    const int32_t* row_lens;  // nullable
    int32_t* out_idx;
    float* out_vals;          // nullable
    void* workspace;          // long rows only (see topk_workspace_bytes)
};

struct BlockTopkParams {
    const float* scores;  // [Hq][Kt][Tq]
    int Hq, Kt, Tq, k;
    int32_t* out_idx;     // [Hq][Tq][k]
    int32_t* out_count;   // [Hq][Tq], nullable
};

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream);

// Fused scorer + top-k: entry point pieces (fused_topk.hip).
size_t logits_topk_workspace_bytes(const LogitsParams& p, int k);
hipError_t launch_logits_topk(const LogitsParams& p, int k, int32_t* out_idx, float* out_vals,
                              void* workspace, size_t ws_bytes, hipStream_t stream);
hipError_t launch_fill_empty_topk(int T, int k, int32_t* out_idx, float* out_vals, hipStream_t stream);
hipError_t launch_block_topk(const BlockTopkParams& p, hipStream_t stream);
hipError_t launch_block_scores(const BlockParams& p, hipStream_t stream);
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);
hipError_t launch_topk_stream(const TopkParams& p, hipStream_t stream);
// Bound on each in-kernel wait of the long-row top-k (polls of its arrival counter);
// when one runs out the row is recomputed by one workgroup.  0 forces that path.
int set_topk_wait_limit(int polls);  // returns the previous bound; < 0 reads it
int topk_stream_cap(int cols, int k);

struct QuantParams {
    const uint16_t* keys;  // [N][key_rs] bf16 bit patterns
    int64_t key_rs;        // elements between key rows
    const int64_t* slots;  // [N]
    uint8_t* k;            // key pages, kp_s bytes apart: [page][64]
    int64_t kp_s;
    uint8_t* ks;           // scale pages, ksp_s bytes apart: [page][4]
    int64_t ksp_s;
    int N, page, num_pages;
    int k_aligned4;        // set by the launcher: k and kp_s allow 4-byte stores
    int keys_aligned16;    // set by the launcher: keys and key_rs allow 16-byte loads
};

hipError_t launch_quantize_store(const QuantParams& p, hipStream_t stream);

// Sparse attention over selected tokens: slot pass.
struct QsaSlotParams {
    const int32_t* ind;     // [rows][ind_rs] logical tokens
    int64_t ind_rs;
    int rows, topk;
    const int32_t* bt;      // [num_req][bt_rs] physical pages
    int64_t bt_rs;
    int num_req, width;
    const int32_t* t2r;     // [rows] request of each row
    int num_blocks, page, ob;
    int32_t* slots;         // [rows][slots_rs]
    int64_t slots_rs;
    int slot_cols;
};

// Sparse attention over selected tokens: decode step.
struct QsaDecodeParams {
    const uint16_t* q;      // bf16 [rows][Hq][128], strides in elements
    int64_t q_rs, q_hs;
    const uint8_t* k;       // e4m3fn cache, byte strides
    const uint8_t* v;
    int64_t bs, ts, khs, vhs;
    const int32_t* slots;
    int64_t slots_rs;
    const int32_t* ind;     // valid count at column topk
    int64_t ind_rs;
    int topk, rows, Hkv, G, ob, num_blocks, page;
    float score_scale;      // softmax_scale * log2(e)
    float out_scale;
    const uint16_t* gate;   // bf16 [rows][Hq][128]
    int64_t gate_rs, gate_hs;
    uint16_t* out;          // bf16 [rows][Hq][128]
    int64_t out_rs, out_hs;
};

hipError_t launch_qsa_slots(const QsaSlotParams& p, hipStream_t stream);
hipError_t launch_qsa_decode(const QsaDecodeParams& p, hipStream_t stream);
size_t topk_workspace_bytes(int rows, int cols, int k);
// leading bytes of that workspace that must be zero when a call starts
size_t topk_workspace_zero_bytes(int rows, int cols, int k);

}  // namespace fp4idx
