/*
 * fp4idx_oracle.c -- plain, slow CPU reference for the FP4 lightning-indexer scorer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is checked
 * against.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the GPU library under
 * sparse_attention_fp4_amd/, and it includes nothing from there.
 *
 * Every function follows the definition on the pages as directly as possible: decode
 * each code to its real value, multiply, add, mask, take the max, sort.  There is no
 * blocking, fusion or reordering.  Sources (cited by page title and section):
 *
 *   [SGL]  "[DSv4.1] Speed up the FP4 indexer scorer by decoding keys without exp2"
 *          (SGLang pull request), sections Modifications and Accuracy Tests.
 *   [M3]   "M3 FP4 Indexer" README, sections 输入 shape 和类型 (input shapes),
 *          输出 shape 和类型 (output shapes), FP4 和 scale layout, 数学语义 (math
 *          semantics) and the causal paragraph that follows it.
 *   [ISS]  "ISSUE -- Lightning Indexer FP4 dequant decodes E2M1 wrong", sections
 *          "Why it's wrong" and "Fix (interim, correct FP32 base)".
 *   [QSA]  vLLM qsa_fp8 API page: _qsa_physical_slots_kernel (invalid pages -> masked),
 *          _decode_slot_layout, _qsa_sparse_paged_decode_kernel and
 *          qsa_sparse_paged_decode (sparse attention over the selected tokens).
 *
 * Precision: every real value is a double.  A per-head dot product of dequantized FP4
 * values is a sum of 128 dyadic terms; orc_dot() adds them in double and reports
 * whether that sum is provably exact (all terms are multiples of 2^L and the sum of
 * their magnitudes stays below 2^(L+53)).  The exact dot is then rounded once to fp32
 * (C's double->float conversion rounds to nearest even).  The weighted head sum is
 * formed in double from the exact dots and rounded once to fp32.
 *
 * Parity status of each function is recorded in the comment above it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MXFP4 0
#define ORC_NVFP4 1

/* ---------------------------------------------------------------------------------
 * Decode of the three code formats.
 * ------------------------------------------------------------------------------- */

/* E2M1 nibble -> value.  The nibble is an index into the level set
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign ([ISS] "Why it's wrong", "Fix
 * (interim...)").  Code 8 is negative zero.  Pinned: the level table printed in [ISS],
 * and the OCP bit-field form (1 exponent-bias, 1 mantissa bit) in the tests. */
double orc_e2m1(unsigned nibble) {
    static const double level[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double mag = level[nibble & 7u];
    return (nibble & 8u) ? -mag : mag;
}

/* E8M0 scale code c -> 2^(c-127), written out literally ([SGL] Modifications: the
 * code is the fp32 exponent field).  Code 255 gives 2^128, which is finite in double
 * and becomes +inf once a product is rounded to fp32.  Pinned against torch's
 * float8_e8m0fnu for codes 0..254. */
double orc_e8m0(unsigned code) {
    return ldexp(1.0, (int)(code & 0xffu) - 127);
}

/* E4M3 (fn variant) scale code -> value, bit by bit: sign bit 7, exponent bits 6..3
 * with bias 7, mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF
 * are NaN; there is no infinity ([M3] FP4 和 scale layout names float8_e4m3fn as the
 * NVFP4 block-scale dtype).  Pinned against torch's float8_e4m3fn for all 256 codes. */
double orc_e4m3(unsigned code) {
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Scale group size S and group count G of a format ([M3] FP4 和 scale layout). */
static int group_size(int fmt) { return fmt == ORC_MXFP4 ? 32 : 16; }
int orc_groups(int fmt) { return fmt == ORC_MXFP4 ? 4 : 8; }

/* One packed 128-element vector (64 bytes, element 2j in the low nibble of byte j,
 * element 2j+1 in the high nibble -- [ISS] "Fix (interim...)", lane 0 = low nibble)
 * with its G scale codes -> 128 real values:  real[d] = E2M1(d) * scale[floor(d/S)]
 * ([M3] 数学语义). */
void orc_dequant_vec(int fmt, const uint8_t* packed, const uint8_t* scales, double* out) {
    int S = group_size(fmt);
    for (int d = 0; d < 128; d++) {
        uint8_t byte = packed[d / 2];
        unsigned nib = (d % 2 == 0) ? (byte & 15u) : (byte >> 4);
        double sc = (fmt == ORC_MXFP4) ? orc_e8m0(scales[d / S]) : orc_e4m3(scales[d / S]);
        out[d] = orc_e2m1(nib) * sc;
    }
}

/* Exponent of the lowest set bit of a finite nonzero double. */
static int lsb_exponent(double x) {
    int e;
    double m = frexp(fabs(x), &e);           /* |x| = m * 2^e, m in [0.5, 1) */
    uint64_t M = (uint64_t)ldexp(m, 53);     /* exact: m has at most 53 bits */
    return e - 53 + __builtin_ctzll(M);
}

/* Dot product of two dequantized 128-vectors, summed in double in index order.
 * Returns 1 when the double sum is provably exact, 0 otherwise (or if a term is not
 * finite).  *abs_sum receives sum_d |q_d k_d| (used as a tolerance base). */
int orc_dot(const double* q, const double* k, double* out, double* abs_sum) {
    double s = 0.0, a = 0.0;
    int lmin = 100000, finite = 1;
    for (int d = 0; d < 128; d++) {
        double t = q[d] * k[d];
        s += t;
        a += fabs(t);
        if (!isfinite(t)) finite = 0;
        else if (t != 0.0) {
            int l = lsb_exponent(t);
            if (l < lmin) lmin = l;
        }
    }
    *out = s;
    if (abs_sum) *abs_sum = a;
    if (!finite) return 0;
    if (a == 0.0) return 1;
    /* each term is an exact product (8-bit significands at most) and a multiple of
     * 2^lmin; every partial sum is then a multiple of 2^lmin bounded by a */
    return a < ldexp(1.0, lmin + 53);
}

/* ---------------------------------------------------------------------------------
 * Weighted-ReLU logits over a paged key cache.
 *
 *   I[t,s] = sum_h w[t,h] * max(q_{t,h} . k_s, 0)       ([ISS] TL;DR; [SGL])
 *
 * Row t belongs to request b when cu_seqlens_q[b] <= t < cu_seqlens_q[b+1].  Key s of
 * request b is token (s mod page) of physical page block_table[b][s / page].  Key s is
 * visible for row t iff s < row_lens[t]; every other column of [0, out_cols) is -inf,
 * whatever the query holds ([SGL] Accuracy Tests: invisible positions stay -inf).  A
 * visible key whose page id is negative or >= num_pages, or whose logical page is past
 * the table width, is treated as invisible ([QSA] slot pass).  Query head h reads key
 * head h / (H / Hkv) ([M3] 数学语义).  max(x, 0) is C's fmax, so a NaN head dot adds 0
 * (the pages say nothing about NaN; fmax is the plain C meaning of max).
 *
 * Layouts (element strides in bytes / elements as noted):
 *   q_fp4   [T][H][64]  bytes, row stride q_rs bytes between rows t (heads contiguous)
 *   q_scale [T][H][G]   bytes, row stride qs_rs bytes
 *   w       [T][H]      float, row stride w_rs floats
 *   k_fp4   [P][Hkv][page][64]  page stride kp_s bytes
 *   k_scale [P][Hkv][page][G]   page stride ksp_s bytes
 *   block_table [B][W] int32, row stride bt_rs elements
 *   logits  [T][out_cols] float, row stride out_rs floats
 *
 * rows / n_rows: optional subset of rows to compute (NULL = all T rows).
 * tolbase (optional, same layout as logits): sum_h |w * max(dot,0)| at each visible
 * position, 0 elsewhere.
 * Returns the number of per-head dots whose double sum was not provably exact.
 * ------------------------------------------------------------------------------- */
long orc_logits_paged(int fmt,
                      const uint8_t* q_fp4, int64_t q_rs,
                      const uint8_t* q_scale, int64_t qs_rs,
                      const float* w, int64_t w_rs,
                      const uint8_t* k_fp4, int64_t kp_s,
                      const uint8_t* k_scale, int64_t ksp_s,
                      const int32_t* block_table, int64_t bt_rs,
                      const int32_t* cu_seqlens_q, const int32_t* row_lens,
                      int T, int B, int H, int Hkv, int page, int num_pages, int W,
                      int out_cols, float* logits, int64_t out_rs, float* tolbase,
                      const int32_t* rows, int n_rows, int n_threads) {
    int G = orc_groups(fmt);
    int R = H / Hkv;
    int nr = rows ? n_rows : T;
    /* the work is shared out by (row, run of ORC_COLS columns) so that a few long rows
     * still keep every thread busy; each output element is computed the same way */
    enum { ORC_COLS = 2048 };
    int n_runs = (out_cols + ORC_COLS - 1) / ORC_COLS;
    long inexact = 0;
    (void)T;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : inexact)
    for (int64_t it = 0; it < (int64_t)nr * n_runs; it++) {
        int ri = (int)(it / n_runs);
        int s_begin = (int)(it % n_runs) * ORC_COLS;
        int s_end = s_begin + ORC_COLS < out_cols ? s_begin + ORC_COLS : out_cols;
        int t = rows ? rows[ri] : ri;
        int b = 0;
        while (b + 1 <= B && cu_seqlens_q[b + 1] <= t) b++;
        if (b >= B) { /* a row outside every request sees nothing */
            for (int s = s_begin; s < s_end; s++) {
                logits[(int64_t)t * out_rs + s] = -INFINITY;
                if (tolbase) tolbase[(int64_t)t * out_rs + s] = 0.0f;
            }
            continue;
        }
        double* qv = (double*)malloc(sizeof(double) * (size_t)H * 128);
        double kv[128];
        for (int h = 0; h < H; h++)
            orc_dequant_vec(fmt, q_fp4 + (int64_t)t * q_rs + (int64_t)h * 64,
                            q_scale + (int64_t)t * qs_rs + (int64_t)h * G, qv + (size_t)h * 128);
        for (int s = s_begin; s < s_end; s++) {
            float* o = logits + (int64_t)t * out_rs + s;
            if (tolbase) tolbase[(int64_t)t * out_rs + s] = 0.0f;
            int visible = s < row_lens[t];
            int lp = s / page, off = s % page;
            int32_t phys = -1;
            if (visible && lp < W) phys = block_table[(int64_t)b * bt_rs + lp];
            if (!visible || phys < 0 || phys >= num_pages) {
                *o = -INFINITY;
                continue;
            }
            double acc = 0.0, tb = 0.0;
            for (int h = 0; h < H; h++) {
                int hk = h / R;
                if (h % R == 0) { /* the first query head of key head hk: decode that key */
                    const uint8_t* kp = k_fp4 + (int64_t)phys * kp_s + ((int64_t)hk * page + off) * 64;
                    const uint8_t* ks = k_scale + (int64_t)phys * ksp_s + ((int64_t)hk * page + off) * G;
                    orc_dequant_vec(fmt, kp, ks, kv);
                }
                double dot, asum;
                if (!orc_dot(qv + (size_t)h * 128, kv, &dot, &asum)) inexact++;
                /* the exact dot rounded once to fp32 is the per-head logit; the weighted
                 * sum uses the exact value.  ReLU is C's fmax(x, 0): a NaN dot (only a
                 * NaN scale code makes one) counts as 0, the pages fix nothing else */
                double r = fmax(dot, 0.0);
                double term = (double)w[(int64_t)t * w_rs + h] * r;
                acc += term;
                tb += fabs(term);
            }
            *o = (float)acc;
            if (tolbase) tolbase[(int64_t)t * out_rs + s] = (float)tb;
        }
        free(qv);
    }
    return inexact;
}

/* ---------------------------------------------------------------------------------
 * Per-head 128-token block-max scores ([M3] 数学语义 and the causal paragraph).
 *
 *   scores[hq][kb][q_global] = max over valid k_local in [128kb, 128kb+128) of
 *                              sum_d Q_real(q_global,hq,d) * K_real(b,k_local,hk,d)
 *
 * q_global = cu_seqlens_q[b] + q_local; k_len[b] = cu_seqlens_k[b+1]-cu_seqlens_k[b];
 * physical_page = kv_indices[cu_page_offsets[b] + kb]; page_row = k_local - 128 kb.
 * k_local is valid iff k_local < k_len[b] and, when causal, k_local <= q_local +
 * offset[b] with offset[b] = qo_offset[b] if given else k_len[b] - q_len[b].  A block
 * with no valid key, or kb >= ceil(k_len[b]/128), is -inf.  Ktiles =
 * ceil(max_seqlen_k / 128).  A physical page id outside [0, num_pages) makes its keys
 * invalid (same reading as for the logits).  The max is C's fmax, so a NaN dot (only a
 * NaN scale code makes one) is skipped, as ReLU skips it in the logits.
 *
 * Layouts: q_fp4 [Tq][Hq][64], q_scale [Tq][Hq][G], k_fp4 [P][Hkv][128][64],
 * k_scale [P][Hkv][128][G], all contiguous; scores [Hq][Ktiles][Tq] float.
 * errbase (optional, same layout as scores): the largest sum_d |q_d k_d| over the
 * valid keys of the block (0 for empty blocks).
 * Returns the number of per-head dots whose double sum was not provably exact.
 * ------------------------------------------------------------------------------- */
long orc_block_scores(int fmt,
                      const uint8_t* q_fp4, const uint8_t* q_scale,
                      const uint8_t* k_fp4, const uint8_t* k_scale,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      const int32_t* cu_page_offsets, const int32_t* kv_indices,
                      const int32_t* qo_offset, int B, int Tq, int Hq, int Hkv, int num_pages,
                      int max_seqlen_k, int causal, float* scores, float* errbase,
                      const int32_t* rows, int n_rows, int n_threads) {
    int G = orc_groups(fmt);
    int R = Hq / Hkv;
    int ktiles = (max_seqlen_k + 127) / 128;
    int nr = rows ? n_rows : Tq;
    long inexact = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : inexact)
    for (int ri = 0; ri < nr; ri++) {
        int qg = rows ? rows[ri] : ri;
        int b = 0;
        while (b + 1 <= B && cu_seqlens_q[b + 1] <= qg) b++;
        if (b >= B) b = B - 1; /* callers guarantee qg < cu_seqlens_q[B] */
        int q_local = qg - cu_seqlens_q[b];
        int q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        int k_len = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
        int offset = qo_offset ? qo_offset[b] : k_len - q_len;
        double qv[128], kv[128];
        for (int hq = 0; hq < Hq; hq++) {
            int hk = hq / R;
            orc_dequant_vec(fmt, q_fp4 + ((int64_t)qg * Hq + hq) * 64,
                            q_scale + ((int64_t)qg * Hq + hq) * G, qv);
            for (int kb = 0; kb < ktiles; kb++) {
                double best = -INFINITY, ebest = 0.0;
                int any = 0;
                if (kb < (k_len + 127) / 128) {
                    int32_t phys = kv_indices[cu_page_offsets[b] + kb];
                    for (int kl = 128 * kb; kl < 128 * kb + 128; kl++) {
                        if (kl >= k_len) continue;
                        if (causal && kl > q_local + offset) continue;
                        if (phys < 0 || phys >= num_pages) continue;
                        int row = kl - 128 * kb;
                        orc_dequant_vec(fmt, k_fp4 + (((int64_t)phys * Hkv + hk) * 128 + row) * 64,
                                        k_scale + (((int64_t)phys * Hkv + hk) * 128 + row) * G, kv);
                        double dot, asum;
                        if (!orc_dot(qv, kv, &dot, &asum)) inexact++;
                        best = fmax(best, dot);   /* a NaN dot is skipped, as in ReLU */
                        if (asum > ebest) ebest = asum;
                        any = 1;
                    }
                }
                int64_t o = ((int64_t)hq * ktiles + kb) * Tq + qg;
                scores[o] = any ? (float)best : -INFINITY;   /* -inf if only NaN dots */
                if (errbase) errbase[o] = (float)ebest;
            }
        }
    }
    return inexact;
}

/* ---------------------------------------------------------------------------------
 * Top-k selection.  For each row, the candidates are the columns s < len (len =
 * row_lens[t] if given, else cols, clipped to cols) whose score is greater than -inf
 * (so -inf and NaN are never selected).  They are ordered by score, larger first, ties
 * broken by the smaller column (the comparisons treat -0 and +0 as equal).  The first min(k, n)
 * are selected and written in increasing column order, then padded with -1 (index) and
 * -inf (value).  A full sort of each row is used.
 * ------------------------------------------------------------------------------- */
typedef struct { float v; int32_t s; } orc_cand;

static int cand_cmp_desc(const void* a, const void* b) {
    const orc_cand* x = (const orc_cand*)a;
    const orc_cand* y = (const orc_cand*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int int_cmp(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

void orc_topk(const float* scores, int64_t row_stride, int rows, int cols,
              const int32_t* row_lens, int k, int32_t* out_idx, float* out_vals,
              int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < rows; t++) {
        int len = row_lens ? row_lens[t] : cols;
        if (len > cols) len = cols;
        if (len < 0) len = 0;
        orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(len > 0 ? len : 1));
        int n = 0;
        for (int s = 0; s < len; s++) {
            float v = scores[(int64_t)t * row_stride + s];
            if (v > -INFINITY) { /* excludes -inf and NaN */
                c[n].v = v;
                c[n].s = s;
                n++;
            }
        }
        qsort(c, (size_t)n, sizeof(orc_cand), cand_cmp_desc);
        int m = n < k ? n : k;
        int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
        for (int i = 0; i < m; i++) sel[i] = c[i].s;
        qsort(sel, (size_t)m, sizeof(int32_t), int_cmp);
        for (int i = 0; i < k; i++) {
            out_idx[(int64_t)t * k + i] = i < m ? sel[i] : -1;
            if (out_vals)
                out_vals[(int64_t)t * k + i] =
                    i < m ? scores[(int64_t)t * row_stride + sel[i]] : -INFINITY;
        }
        free(sel);
        free(c);
    }
}

/* Threads an OpenMP region would use (for reporting). */
/* ---------------------------------------------------------------------------------
 * MXFP4 quantize-and-store of index keys into the paged cache.
 *
 * [SGL] bench and Modifications: keys [N][128] in bf16 are written into 64-byte
 * nibble rows and 4 E8M0 codes per token of a paged cache, at the page and token a
 * slot names (page = slot / page_size, token = slot % page_size); rounding is to
 * nearest even ("rne=True"); stored exponent codes are clamped to 1..254.  [ISS] "Why
 * it's wrong": the stored nibble is the index into {0, 0.5, 1, 1.5, 2, 3, 4, 6} with
 * the sign in bit 3.
 *
 * Reading (the pages do not say how a block's exponent is chosen): the OCP
 * microscaling rule -- the scale of a 32-value block is 2^(floor(log2(amax)) - 2),
 * with 2 the exponent of E2M1's largest value 6, so amax / scale lies in [4, 8); the
 * code is that exponent + 127 clamped to 1..254 (an all-zero block gets code 1).  Each
 * value is divided by the scale and mapped to the nearest of the eight magnitudes,
 * ties going to the even index (mantissa bit 0); magnitudes above 6 take 6; the sign
 * bit is copied (so -0 and small negatives that round to zero store code 8).
 * Parity pinned by closed forms, a hand-worked fixture and properties in the tests.
 * ------------------------------------------------------------------------------- */

/* One block of 32 values -> 16 packed bytes (element 2j in the low nibble of byte j)
 * and its E8M0 code. */
void orc_quantize_mx_block(const double* x, uint8_t* packed, uint8_t* code_out) {
    static const double level[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double amax = 0.0;
    for (int i = 0; i < 32; i++)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    int code = 1;
    if (amax > 0.0) {
        int e;
        frexp(amax, &e);             /* amax = f * 2^e with f in [0.5, 1) */
        int shared = (e - 1) - 2;    /* floor(log2(amax)) - 2 */
        code = shared + 127;
        if (code < 1) code = 1;
        if (code > 254) code = 254;
    }
    double scale = ldexp(1.0, code - 127);
    for (int i = 0; i < 32; i++) {
        double m = fabs(x[i]) / scale;
        int best = 0;
        for (int c = 1; c < 8; c++) {
            double d = fabs(m - level[c]), db = fabs(m - level[best]);
            if (d < db || (d == db && (c & 1) == 0)) best = c;
        }
        unsigned nib = (unsigned)best | (signbit(x[i]) ? 8u : 0u);
        if (i & 1) packed[i >> 1] = (uint8_t)(packed[i >> 1] | (nib << 4));
        else packed[i >> 1] = (uint8_t)nib;
    }
    *code_out = (uint8_t)code;
}

/* Keys [N][128] (as doubles) into the cache: token n goes to slot slots[n]; a slot
 * outside [0, num_pages * page) is skipped.  Layouts as in orc_logits_paged (one key
 * head): k_fp4 pages k_page_stride bytes apart holding [page][64], k_scale pages
 * ks_page_stride bytes apart holding [page][4]. */
void orc_quantize_store(const double* keys, const int64_t* slots, int N,
                        uint8_t* k_fp4, int64_t k_page_stride,
                        uint8_t* k_scale, int64_t ks_page_stride,
                        int page, int num_pages) {
    for (int n = 0; n < N; n++) {
        int64_t slot = slots[n];
        if (slot < 0 || slot >= (int64_t)num_pages * page) continue;
        int64_t pg = slot / page, tok = slot % page;
        for (int g = 0; g < 4; g++)
            orc_quantize_mx_block(keys + (int64_t)n * 128 + 32 * g,
                                  k_fp4 + pg * k_page_stride + tok * 64 + 16 * g,
                                  k_scale + pg * ks_page_stride + tok * 4 + g);
    }
}

int orc_max_threads(int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) return n_threads;
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------
 * Sparse paged attention over the selected tokens ([QSA] vLLM qsa_fp8 API page):
 * the consumer of a top-k token selection.  Two steps: the slot pass turns each
 * row's logical token indices into physical cache slots; the decode step attends
 * from every query head over the selected tokens of its KV head.
 * ------------------------------------------------------------------------------- */

/* Bits that hold a token's place inside its page in a slot: the bit length of
 * page_size - 1, and at least 1 ([QSA] _decode_slot_layout).  Pinned by closed forms
 * in the tests. */
int orc_qsa_offset_bits(int page_size) {
    int b = 0;
    while (b < 31 && ((int64_t)1 << b) < (int64_t)page_size) b++;
    return b < 1 ? 1 : b;
}

/* Slot pass ([QSA] _qsa_physical_slots_kernel and qsa_sparse_paged_decode).
 *
 * Row r belongs to request b = token_to_req[r].  For column c < topk, the logical
 * token x = indices[r][c] sits at place x % page_size of logical page x / page_size,
 * whose physical page p is block_table[b][x / page_size].  The slot is
 * (p << offset_bits) | (x % page_size) when 0 <= b < num_requests, x >= 0,
 * x / page_size < table_width and 0 <= p < num_cache_blocks; otherwise it is -1.
 * Columns topk .. slot_cols-1 are -1 (padding).  The valid count stored in column
 * topk of indices is not read here (the decode step reads it).
 * Layouts: indices [rows][>= topk] int32 (row stride ind_rs), block_table
 * [num_requests][table_width] int32 (row stride bt_rs), slots [rows][slot_cols] int32
 * (row stride slots_rs).  Parity pinned by a hand-worked table in the tests. */
void orc_qsa_slots(const int32_t* indices, int64_t ind_rs, int rows, int topk,
                   const int32_t* block_table, int64_t bt_rs, int num_requests,
                   int table_width, const int32_t* token_to_req, int num_cache_blocks,
                   int page_size, int32_t* slots, int64_t slots_rs, int slot_cols) {
    int ob = orc_qsa_offset_bits(page_size);
    for (int r = 0; r < rows; r++) {
        int b = token_to_req[r];
        for (int c = 0; c < slot_cols; c++) {
            int32_t slot = -1;
            if (c < topk && b >= 0 && b < num_requests) {
                int32_t x = indices[(int64_t)r * ind_rs + c];
                if (x >= 0 && x / page_size < table_width) {
                    int32_t p = block_table[(int64_t)b * bt_rs + x / page_size];
                    if (p >= 0 && p < num_cache_blocks)
                        slot = (int32_t)(((uint32_t)p << ob) | (uint32_t)(x % page_size));
                }
            }
            slots[(int64_t)r * slots_rs + c] = slot;
        }
    }
}

/* bf16 bit pattern -> value (the 16 bits are the top half of an IEEE binary32). */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Decode step ([QSA] _qsa_sparse_paged_decode_kernel, qsa_sparse_paged_decode):
 * grouped-query attention of each row over its selected tokens.
 *
 * Row r selects the columns c < min(count, topk), count = indices[r][topk], whose slot
 * is not negative (reading: a column at or past the valid count is not selected even
 * when its slot is valid; a negative count selects nothing).  Selected token j lives at
 * place slot & (2^offset_bits - 1) of cache page slot >> offset_bits.  Query head h
 * uses KV head g = h / (Hq / Hkv).  With K_j, V_j the e4m3fn codes of token j, head g
 * decoded exactly (orc_e4m3) and q, gate the bf16 values:
 *
 *   s_j      = softmax_scale * sum_d q[r][h][d] * K_j[d]
 *   a_j      = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i)
 *   out[r][h][d] = output_scale * (sum_j a_j V_j[d]) * sigmoid(gate[r][h][d])
 *
 * and out = 0 when nothing is selected ([QSA] epilogue: rows with no probability mass
 * output zero).  A token selected twice counts twice.  Everything is computed in double
 * from exact decodes; the page's own kernel rounds the probabilities to fp16 and the
 * output to bf16, which the tests allow for in their tolerance.
 * Layouts: q and gate [rows][Hq][D] bf16 bits with row / head strides in elements;
 * K and V cache token (page p, place t, head g) at byte p*block_stride +
 * t*token_stride + g*head_stride (separate head strides for K and V); out [rows][Hq][D]
 * double, contiguous.  tolbase (optional, same layout as out): output_scale *
 * sum_j a_j |V_j[d]| * sigmoid(gate), the size of the terms the output sums.
 * Parity pinned in the tests by closed forms (one token, equal keys, a two-token
 * case with weights 3/4 and 1/4), invariants (order, masking, duplicates) and by
 * torch's scaled_dot_product_attention in double on the gathered tokens. */
void orc_qsa_decode(const uint16_t* q, int64_t q_rs, int64_t q_hs,
                    const uint8_t* k_cache, const uint8_t* v_cache, int64_t block_stride,
                    int64_t token_stride, int64_t k_head_stride, int64_t v_head_stride,
                    const int32_t* slots, int64_t slots_rs,
                    const int32_t* indices, int64_t ind_rs, int topk,
                    int rows, int Hq, int Hkv, int D, int offset_bits,
                    double softmax_scale, double output_scale,
                    const uint16_t* gate, int64_t gate_rs, int64_t gate_hs,
                    double* out, double* tolbase, int n_threads) {
    int G = Hq / Hkv;
    int32_t mask = (int32_t)((1u << offset_bits) - 1u);
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; r++) {
        int n = indices[(int64_t)r * ind_rs + topk];
        if (n > topk) n = topk;
        if (n < 0) n = 0;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int* sel = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
        int m = 0;
        for (int c = 0; c < n; c++)
            if (slots[(int64_t)r * slots_rs + c] >= 0) sel[m++] = c;
        for (int h = 0; h < Hq; h++) {
            int g = h / G;
            const uint16_t* qh = q + (int64_t)r * q_rs + (int64_t)h * q_hs;
            double smax = -INFINITY;
            for (int j = 0; j < m; j++) {
                int32_t slot = slots[(int64_t)r * slots_rs + sel[j]];
                const uint8_t* kr = k_cache + (int64_t)(slot >> offset_bits) * block_stride +
                                    (int64_t)(slot & mask) * token_stride +
                                    (int64_t)g * k_head_stride;
                double acc = 0.0;
                for (int d = 0; d < D; d++) acc += bf16_value(qh[d]) * orc_e4m3(kr[d]);
                s[j] = softmax_scale * acc;
                if (s[j] > smax) smax = s[j];
            }
            double z = 0.0;
            for (int j = 0; j < m; j++) {
                s[j] = exp(s[j] - smax);
                z += s[j];
            }
            for (int d = 0; d < D; d++) {
                double o = 0.0, a = 0.0;
                for (int j = 0; j < m; j++) {
                    int32_t slot = slots[(int64_t)r * slots_rs + sel[j]];
                    const uint8_t* vr = v_cache + (int64_t)(slot >> offset_bits) * block_stride +
                                        (int64_t)(slot & mask) * token_stride +
                                        (int64_t)g * v_head_stride;
                    double v = orc_e4m3(vr[d]);
                    o += s[j] * v;
                    a += s[j] * fabs(v);
                }
                double gv = bf16_value(gate[(int64_t)r * gate_rs + (int64_t)h * gate_hs + d]);
                double sig = 1.0 / (1.0 + exp(-gv));
                int64_t at = ((int64_t)r * Hq + h) * D + d;
                out[at] = m > 0 ? output_scale * (o / z) * sig : 0.0;
                if (tolbase) tolbase[at] = m > 0 ? fabs(output_scale) * (a / z) * sig : 0.0;
            }
        }
        free(sel);
        free(s);
    }
}
