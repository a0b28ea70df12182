/*
 * fp4idx.h -- C ABI of libfp4idx.so, the FP4 lightning-indexer scorer for MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [SGL] "[DSv4.1] Speed up the FP4 indexer scorer by decoding keys without exp2"
 *         (SGLang pull request): Motivation (the paged scorer and its tile),
 *         Modifications (E2M1 and E8M0 decode), Accuracy Tests (invisible positions are
 *         -inf; metadata is read at replay time), and the bench script (4 verify rows,
 *         shuffled 64-token pages, a request table mapping tokens to pages).
 *   [M3]  "M3 FP4 Indexer" README: 公共约束 (constraints), 输入 shape 和类型 (input shapes),
 *         输出 shape 和类型 (output shape), FP4 和 scale layout, 数学语义 (math semantics)
 *         and the causal paragraph after it.
 *   [ISS] "ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong": TL;DR (the score
 *         I[t,s]), "Fix (interim...)" (E2M1 level set, low nibble first), "Fix
 *         (production target)" (ReLU and head weights in the epilogue, wave-level top-k).
 *   [QSA] vLLM qsa_fp8 API page, _qsa_physical_slots_kernel: an entry that names no valid
 *         page is masked; -1 pads a selection.  _decode_slot_layout,
 *         _qsa_sparse_paged_decode_kernel and qsa_sparse_paged_decode: the slot pass and
 *         the sparse attention over the selected tokens of an fp8 e4m3fn K/V cache.
 *
 * Conventions for every entry point
 *   - Every pointer is device memory owned by the caller, except where a parameter says
 *     otherwise.  The library allocates nothing, keeps no state between calls and
 *     never copies device data to the host.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and the call returns without waiting.  Device metadata (sequence
 *     lengths, tables) is read by the kernels when they run, so the calls may be
 *     captured in a hipGraph and replayed with new metadata in the same buffers.
 *   - Argument errors are detected on the host from the scalar arguments and the
 *     pointer values only.  On error nothing is enqueued and a nonzero FP4IDX_E* code
 *     is returned; fp4idx_strerror() names it.
 *   - Packed FP4: 64 bytes hold 128 E2M1 values; element 2j is the low nibble of byte
 *     j and element 2j+1 its high nibble; nibble bit 3 is the sign and bits 2..0 index
 *     the levels {0, 0.5, 1, 1.5, 2, 3, 4, 6} [ISS].
 *   - Block scales [M3 FP4 和 scale layout]: MXFP4 = one E8M0 code per 32 values (G=4),
 *     value 2^(code-127); NVFP4 = one E4M3 (fn) code per 16 values (G=8), with no
 *     tensor-level global scale.  real[d] = E2M1[d] * scale[floor(d / S)].  E8M0 codes
 *     0 and 255 are outside the stored range 1..254 [SGL Modifications]; what they give
 *     is not specified (a code-255 scale makes the matrix core return NaN, and an MXFP4
 *     logit that holds such a head dot is NaN).  Every stored code 1..254 and every
 *     E4M3 code is decoded exactly.
 *   - NaN: a NaN head dot (only a NaN E4M3 scale code, or the E8M0 code 255 above, can
 *     make one) counts as 0 in the NVFP4 ReLU and is skipped by the block maxima; top-k
 *     never selects NaN.
 */
#ifndef FP4IDX_H
#define FP4IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* block-scale formats */
enum { FP4IDX_MXFP4 = 0, FP4IDX_NVFP4 = 1 };

/* status codes */
enum {
    FP4IDX_OK = 0,
    FP4IDX_EINVAL = 1,       /* null required pointer, bad dimension, bad format, ... */
    FP4IDX_EUNSUPPORTED = 2, /* a valid request the library does not implement */
    FP4IDX_EALIGN = 3,       /* a pointer or stride that must be 16-byte aligned is not */
    FP4IDX_EHIP = 4,         /* the HIP runtime reported an error at launch */
    FP4IDX_EWORKSPACE = 5    /* workspace missing or smaller than required */
};

/* Weighted-ReLU indexer logits over a paged key cache [ISS TL;DR; SGL]:
 *
 *     logits[t][s] = sum_{h<H} w[t][h] * max(q[t][h] . k_b(t)[hk(h)][s], 0)
 *
 * for s < row_lens[t], and -inf for every other s in [0, out_cols) whatever the query
 * holds [SGL Accuracy Tests].  Row t belongs to request b(t), the b with
 * cu_seqlens_q[b] <= t < cu_seqlens_q[b+1].  Logical key s of request b is token
 * (s % page_size) of physical page block_table[b * bt_row_stride + s / page_size]; a
 * visible key whose logical page is >= table_width or whose page id is outside
 * [0, num_pages) is scored -inf [QSA].  Query head h reads key head hk(h) = h / (H/Hkv)
 * [M3 数学语义].
 *
 * Layouts (strides in bytes for byte arrays, in elements otherwise):
 *   q_fp4   [T][H][64] uint8     rows t are q_row_stride bytes apart; heads contiguous
 *   q_scale [T][H][G]  uint8     rows qs_row_stride bytes apart
 *   w       [T][H]     float     rows w_row_stride floats apart (non-contiguous rows
 *                                of q/w are allowed [SGL Accuracy Tests])
 *   k_fp4   [P][Hkv][page_size][64] uint8, pages k_page_stride bytes apart
 *   k_scale [P][Hkv][page_size][G]  uint8, pages ks_page_stride bytes apart.  A combined
 *           page (values then scales, [SGL] bench) is k_scale = k_fp4 + Hkv*page_size*64
 *           with both page strides = Hkv*page_size*(64+G).
 *   block_table [B][table_width] int32 (rows bt_row_stride apart), -1 = no page
 *   cu_seqlens_q [B+1] int32, nondecreasing, cu_seqlens_q[0] = 0, cu_seqlens_q[B] <= T;
 *           a row t >= cu_seqlens_q[B] belongs to no request and is -inf everywhere
 *   row_lens [T] int32
 *   logits [T][out_cols] float, rows out_row_stride floats apart
 * Alignment: q_fp4, k_fp4, k_scale and their row/page strides must be multiples of 16
 * bytes (EALIGN).
 * Limits: H % Hkv == 0, page_size in {64, 128} (else EUNSUPPORTED), 1 <= H <= 128,
 * out_row_stride <= 2^27 floats (else EUNSUPPORTED).
 * fmt = FP4IDX_MXFP4 or FP4IDX_NVFP4. */
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
                        void* stream);

/* Weighted-ReLU logits and their top-k in one call, without writing the logits [ISS
 * "Fix (production target)": scores on the matrix cores, ReLU and head weights in the
 * epilogue, the top-k selected without a serial heap].  The result is exactly that of
 * fp4idx_topk over the logits fp4idx_logits_paged would write with the same arguments
 * (out_cols columns): per row t, the k largest finite scores of the visible columns
 * (ties to the smaller column), out_idx[t][0..m) = their columns in increasing order,
 * m = min(k, #finite visible scores), out_idx[t][m..k) = -1; out_vals (nullable) the
 * scores, -inf padded.  The logits arguments mean what they mean for
 * fp4idx_logits_paged.
 * How: the scores of every 16th page give each row a threshold that about 2k scores
 * of the row reach; the scorer then keeps only scores at or above it, and the exact
 * selection runs over those.  A row where fewer than k scores reach the threshold is
 * scored again keeping every score, so the result never depends on the sample.  With
 * fewer than 512 rows the logits are written into the workspace instead and the plain
 * top-k (fp4idx_topk) selects from them: the same result, faster for few rows.
 * workspace: fp4idx_logits_topk_workspace_bytes(...) bytes, 256-byte aligned,
 * caller-owned device memory (contents need no initialisation; calls that run
 * concurrently must not share one).  With 512 rows or more only the kept scores
 * (about 2k per row) are written there, plus the sampled scores (1/16 of the columns).
 * Limits: 1 <= k <= 2048 and out_cols <= 2^24 (else EUNSUPPORTED); the logits limits
 * otherwise; EWORKSPACE when the workspace is missing, short or misaligned. */
size_t fp4idx_logits_topk_workspace_bytes(int fmt, int T, int B, int H, int Hkv, int page_size,
                                          int table_width, int out_cols, int k);
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
                             void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free fp4idx_logits_topk_paged, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments and result, without the workspace.  Its scratch is one
 * static array of FP4IDX_NOALLOC_SCRATCH_BYTES in the library's code object on each
 * GPU (reserved when the library is first used on that GPU, held until the process
 * ends); the call allocates nothing.  The stream must belong to the current device.
 * A request whose fp4idx_logits_topk_workspace_bytes(...) exceeds that size returns
 * FP4IDX_EWORKSPACE before anything is enqueued (4 rows of 400k columns, or 64 rows of
 * 131072, fit; long prefills do not).  Every call on one GPU uses the same array, so
 * calls that overlap on one GPU (other streams, other threads) race: the caller
 * serialises them.  What must start zeroed is cleared by each call's own kernels. */
#define FP4IDX_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
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
                                     int32_t* out_idx, float* out_vals, void* stream);

/* Per-head 128-token block-max scores [M3 数学语义]:
 *
 *     scores[hq][kb][q] = max over valid k_local in [128 kb, 128 kb + 128) of
 *                         q[q][hq] . k[kv_indices[cu_page_offsets[b] + kb]][hq/(Hq/Hkv)][k_local-128kb]
 *
 * for query token q = cu_seqlens_q[b] + q_local of batch item b.  k_local is valid iff
 * k_local < k_len[b] = cu_seqlens_k[b+1] - cu_seqlens_k[b], the page id is in
 * [0, num_pages), and, when causal, k_local <= q_local + offset[b] with offset[b] =
 * qo_offset[b] if qo_offset is given, else k_len[b] - q_len[b] (bottom-right).  A
 * block with no valid key, and every kb >= ceil(k_len[b] / 128), is -inf.  No ReLU and
 * no weights.
 *
 * Layouts (all contiguous): q_fp4 [Tq][Hq][64], q_scale [Tq][Hq][G], k_fp4
 * [num_pages][Hkv][128][64], k_scale [num_pages][Hkv][128][G]; cu_seqlens_q,
 * cu_seqlens_k, cu_page_offsets [B+1] int32 (prefix sums from 0; batch b owns logical
 * pages [cu_page_offsets[b], cu_page_offsets[b+1]) = ceil(k_len[b]/128) of them);
 * kv_indices [cu_page_offsets[B]] int32; qo_offset [B] int32 or NULL; scores
 * [Hq][Ktiles][Tq] float with Ktiles = ceil(max_seqlen_k / 128).
 * Caller guarantees [M3 输入 shape 和类型]: every q_len[b] <= max_seqlen_q and every
 * k_len[b] <= max_seqlen_k.
 * Errors: EINVAL for max_seqlen_q <= 0, Hq % Hkv != 0, qo_offset given with causal == 0,
 * or a bad fmt; EALIGN for q_fp4 / k_fp4 / k_scale not 16-byte aligned. */
int fp4idx_block_scores(int fmt,
                        const uint8_t* q_fp4, const uint8_t* q_scale,
                        const uint8_t* k_fp4, const uint8_t* k_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* cu_page_offsets, const int32_t* kv_indices,
                        const int32_t* qo_offset,
                        int B, int Tq, int Hq, int Hkv, int num_pages,
                        int max_seqlen_q, int max_seqlen_k, int causal,
                        float* scores, void* stream);

/* Top-k 128-token blocks of every (head, query) from block scores [M3 public API: the
 * block-score interface returns no TopK; a caller takes it along the Ktiles dimension]:
 * for head h and query q, the candidates are the blocks kb < Ktiles whose score
 * scores[h][kb][q] is greater than -inf (-inf and NaN are never chosen); the k largest
 * are chosen, ties toward the smaller block (-0 equals +0).
 * out_idx[h][q][0..m) receives the chosen blocks in increasing order, m = min(k,
 * #candidates), and out_idx[h][q][m..k) = -1; out_count[h][q] (nullable) receives m.
 * scores: [Hq][Ktiles][Tq] float, contiguous (the layout fp4idx_block_scores writes);
 * out_idx: [Hq][Tq][k] int32; out_count: [Hq][Tq] int32; all caller-owned device
 * memory.  Asynchronous on `stream`; nothing is allocated.
 * Limits: 1 <= k <= 64 (else EUNSUPPORTED); EINVAL for Hq < 1, Ktiles < 0, Tq < 0,
 * k < 1 or a missing pointer. */
int fp4idx_block_topk(const float* scores, int Hq, int Ktiles, int Tq, int k,
                      int32_t* out_idx, int32_t* out_count, void* stream);

/* Bytes of device workspace fp4idx_topk needs for these sizes (0 if none). */
size_t fp4idx_topk_workspace_bytes(int rows, int cols, int k);

/* Top-k selection over score rows [ISS "Fix (production target)"]: for each row t, the
 * candidates are the columns s < len(t) (len = min(row_lens[t], cols) if row_lens is
 * given, else cols) whose score is greater than -inf (-inf and NaN are never selected).
 * The k largest are selected, ties broken toward the smaller column (-0 equals +0).
 * out_idx[t][0..m) receives the selected columns in increasing order, m = min(k,
 * #candidates), and out_idx[t][m..k) = -1 [QSA].  out_vals (nullable) receives the
 * matching scores, -inf in the padding.
 * scores: [rows][row_stride] float (row_stride >= cols); out_idx, out_vals: [rows][k].
 * workspace: device memory of at least fp4idx_topk_workspace_bytes(rows, cols, k),
 * 256-byte aligned, owned by the caller (NULL allowed when that size is 0: rows of at
 * most 8192 columns, or of at most 32768 columns when there are more than 64 rows, need
 * none).  It carries per-row histograms and arrival counters between the kernels, or
 * the workgroups, of one call: it must be zero-filled before its first use, and every
 * call that returns FP4IDX_OK leaves it ready for the next one with the same rows and
 * cols (also under graph replay).  Its layout depends on both, so memory that served
 * another shape must be zero-filled again first, and so must a workspace after a call
 * that returns FP4IDX_EHIP (a launch failed part way).  Calls that run concurrently
 * must not share a workspace.
 * Limits: 1 <= k <= 8192 and cols <= 524288 (else EUNSUPPORTED). */
int fp4idx_topk(const float* scores, int64_t row_stride, int rows, int cols,
                const int32_t* row_lens, int k,
                int32_t* out_idx, float* out_vals,
                void* workspace, size_t workspace_bytes, void* stream);

/* For up to 64 rows of 8193..53248 columns (when the GPU's dies can hold every row's
 * chunk workgroups at once: up to 16 rows of 53248 columns, 32 of 32768, 64 of 16384)
 * and for many rows of up to 131072 columns (more than 512 chunks of 4096 columns in
 * all; up to 32 rows, or 48 to 64), fp4idx_topk
 * (and the few-rows route of fp4idx_logits_topk_paged) runs one kernel whose workgroups
 * wait for each other in memory.  Each such wait polls at most `polls` times (default 65536, about 30 ms or
 * more); a wait that runs out -- the row's workgroups could not all run at once, e.g.
 * beside other work on the GPU -- has one workgroup recompute the row from its scores:
 * the same result, later.  0 forces that path (for tests).  Sets the bound for later
 * launches from this process and returns the previous one; negative values leave it
 * unchanged. */
int fp4idx_set_topk_wait_limit(int polls);

/* MXFP4 quantize-and-store of index keys into the paged cache ([SGL] Modifications and
 * bench: bf16 keys become E2M1 nibbles plus one E8M0 code per 32 values, rounded to
 * nearest even, written at the page and token their slot names; stored exponent codes
 * are clamped to 1..254; [ISS] "Why it's wrong": nibble = index into the level set,
 * sign in bit 3):
 *
 *     token n (keys row n, 128 values) -> page slots[n] / page_size,
 *                                         token slots[n] % page_size
 *
 * Each block of 32 values gets the scale 2^(floor(log2(amax)) - 2), with amax its
 * largest magnitude (the OCP microscaling rule; the pages do not say how the exponent
 * is chosen); its E8M0 code is that exponent + 127 clamped to 1..254 (an all-zero or
 * subnormal block gets 1).  Each value divided by the scale is stored as the nearest
 * level, ties to the even index, magnitudes above 6 as 6, with its sign bit copied
 * (so -0 stores 8).  Keys must be finite (NaN and Inf give unspecified codes).
 *
 * Layouts: keys [N][key_row_stride] bf16 bit patterns (row stride in elements, even;
 * keys 4-byte aligned, else EALIGN); slots [N] int64 -- a slot outside
 * [0, num_pages * page_size) leaves its token unwritten; k_fp4 / k_scale: the cache of
 * fp4idx_logits_paged with Hkv = 1 (MXFP4: [P][page_size][64] nibbles and [P][page_size][4]
 * codes, pages k_page_stride / ks_page_stride bytes apart).  Two tokens with the same
 * slot race.  Limits: page_size in {64, 128} (else EUNSUPPORTED). */
int fp4idx_quantize_store_k(const uint16_t* keys, int64_t key_row_stride,
                            const int64_t* slots, int N,
                            uint8_t* k_fp4, int64_t k_page_stride,
                            uint8_t* k_scale, int64_t ks_page_stride,
                            int page_size, int num_pages, void* stream);

/* Slot pass of the sparse attention over selected tokens [QSA _qsa_physical_slots_kernel,
 * _decode_slot_layout]: row r of request b = token_to_req[r]; for column c < topk the
 * logical token x = indices[r][c] sits at place x % page_size of logical page
 * x / page_size, whose physical page is p = block_table[b][x / page_size];
 *   slots[r][c] = (p << offset_bits) | (x % page_size),
 * offset_bits = the bit length of page_size - 1, at least 1, when 0 <= b < num_requests,
 * x >= 0, x / page_size < table_width and 0 <= p < num_cache_blocks; otherwise -1.
 * Columns topk .. slot_cols-1 are -1.  The slots serve every KV head.
 * Layouts: indices [rows][>= topk] int32 (row stride in elements; the valid count that
 * fp4idx_qsa_decode reads sits at column topk), block_table [num_requests][table_width]
 * int32 (row stride in elements), token_to_req [rows] int32, slots [rows][slot_cols]
 * int32 (row stride in elements); all caller-owned device memory.
 * Errors: EINVAL for rows < 0, topk < 1, slot_cols < topk, page_size < 1,
 * num_requests < 1, table_width < 1, num_cache_blocks < 1, strides shorter than a row,
 * a missing pointer, or (num_cache_blocks << offset_bits) >= 2^31 (a slot must fit in
 * int32). */
int fp4idx_qsa_slots(const int32_t* indices, int64_t indices_row_stride, int rows, int topk,
                     const int32_t* block_table, int64_t block_table_row_stride,
                     int num_requests, int table_width, const int32_t* token_to_req,
                     int num_cache_blocks, int page_size,
                     int32_t* slots, int64_t slots_row_stride, int slot_cols, void* stream);

/* Sparse grouped-query attention over the selected tokens [QSA
 * _qsa_sparse_paged_decode_kernel, qsa_sparse_paged_decode].  Row r selects the columns
 * c < min(max(indices[r][topk], 0), topk) whose slot is not -1 and names a page below
 * num_cache_blocks (a column at or past the valid count is never selected).  Query head
 * h reads KV head g = h / (Hq / Hkv).  With K_j, V_j the e4m3fn codes of selected token j
 * (page slot >> offset_bits, place slot & (2^offset_bits - 1)) and q, gate bf16:
 *   s_j = softmax_scale * q[r][h] . K_j          (bf16 x e4m3 products, fp32 sums)
 *   a_j = softmax over the selected j            (probabilities rounded to fp16 for the
 *                                                  product with V, fp32 normalizer)
 *   out[r][h][d] = bf16(bf16(output_scale * sum_j a_j V_j[d]) * sigmoid(gate[r][h][d]))
 * and out = 0 for a row with nothing selected.  A token selected twice counts twice.
 * Layouts: q, gate, out [rows][Hq][head_dim] bf16 (uint16 bit patterns) with row and head
 * strides in elements, dims contiguous; the caches hold token (page p, place t, head g) at
 * byte p * block_stride + t * token_stride + g * k_head_stride (v_head_stride for V), dims
 * contiguous (one combined cache with V at k_cache + head_dim is fine); slots as written
 * by fp4idx_qsa_slots (>= min(count, topk) columns per row); indices as above.  All
 * caller-owned device memory; asynchronous on `stream`; nothing is allocated.
 * Limits: head_dim == 128 and 1 <= Hq / Hkv <= 16 (else EUNSUPPORTED); block_stride and
 * token_stride below 2^32 (else EUNSUPPORTED); EALIGN unless q, gate, out, k_cache and
 * v_cache are 16-byte aligned, the bf16 strides are multiples of 8 elements and the
 * cache strides multiples of 16 bytes; EINVAL for rows < 0, topk < 1, Hkv < 1,
 * Hq % Hkv != 0, page_size < 1, num_cache_blocks < 1, a missing pointer, or
 * (num_cache_blocks << offset_bits) >= 2^31. */
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
                      void* stream);

/* Static string naming a status code. */
const char* fp4idx_strerror(int code);

/* Library ABI version (major * 100 + minor). */
int fp4idx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4IDX_H */
