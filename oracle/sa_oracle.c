/*
 * sa_oracle.c -- plain, slow CPU oracle for index-selected sparse attention over a paged
 * KV cache (indexer scores -> Top-K -> sparse attention).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library. It shares no code, header, table or constant with the HIP library
 * and includes none of its files. Every loop below is the plain definition of the step it
 * computes, in the order the definition states it; nothing is blocked, fused or reordered.
 *
 * Pages cited (by title and section):
 *   [SameDay]  "How the Ascend Computing Platform Achieves Same-Day Inference Adaptation for
 *              Ultra-Large Sparse Models"
 *   [Domestic] "Engineering Path for Day-0 Adaptation of Trillion-Scale Sparse Models on
 *              Domestic AI Accelerators"
 *   [CANN]     "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on
 *              Huawei Ascend CANN Architecture"
 *   [GPUGuide] "Adapting GPU Software Stacks for Ultra-Large-Scale Sparse Attention Models:
 *              A Day-0 Engineering Guide"
 *
 * Arithmetic: REAL is double unless built with -DORACLE_FLOAT (then float). Inputs arrive in
 * their storage formats (bf16 bit patterns, OCP E4M3 codes) and are decoded here from the
 * formats' own definitions.
 *
 * Return codes: 0 = ok, 1 = an input violates the stated preconditions (nothing is written
 * past the first violation, results are then undefined).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_FLOAT
typedef float REAL;
#define ORACLE_REAL_BYTES 4
#else
typedef double REAL;
#define ORACLE_REAL_BYTES 8
#endif

int ora_real_bytes(void) { return ORACLE_REAL_BYTES; }

/* Threads the OpenMP loops below run with (for reporting timings). */
#ifdef _OPENMP
#include <omp.h>
int ora_max_threads(void) { return omp_get_max_threads(); }
#else
int ora_max_threads(void) { return 1; }
#endif

/* ---------------------------------------------------------------- storage formats */

/* bf16 is the upper half of an IEEE-754 binary32 word: widen by appending 16 zero bits. */
REAL ora_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (REAL)f;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits, subnormals when the exponent field is 0, no infinities, S.1111.111 is NaN.
 * Quantized data types for the indexer and the KV cache: [CANN] §2.1 and §3. */
REAL ora_e4m3(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    REAL mag;
    if (e == 15 && m == 7) return (REAL)NAN;
    if (e == 0)
        mag = (REAL)m / 8 * ldexp(1.0, 1 - 7);       /* subnormal: 0.m x 2^(1-bias) */
    else
        mag = (1 + (REAL)m / 8) * ldexp(1.0, e - 7); /* normal: 1.m x 2^(e-bias) */
    return sign ? -mag : mag;
}

/* Nearest E4M3 code to y, ties to the code with an even mantissa, saturating at +-448 (the
 * largest finite magnitude; the format has no infinities). The sign bit is y's sign bit, so
 * -0.0 and negative values that round to zero give 0x80. The search simply visits every
 * finite non-negative code. */
uint8_t ora_e4m3_encode(double y) {
    double a = fabs(y);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double err = fabs((double)ora_e4m3((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    if (a > 448.0) best = 0x7E;
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* MXFP8 (the OCP microscaling format with E4M3 elements): a block of 32 consecutive elements
 * shares one power-of-two scale 2^X, stored as the E8M0 byte X + 127. The shared exponent is
 *     X = floor(log2(amax)) - 8        (8 = the exponent of E4M3's largest power of two)
 * clamped to [-127, 127], with X = -127 for an all-zero block; each element is encoded as
 * E4M3(v / 2^X) with saturation. The indexer runs in this format, with per-group dynamic
 * quantization and a group of 32: [CANN] §3. */
int ora_mx_exponent(double amax) {
    if (!(amax > 0)) return -127;
    int e;
    frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1 */
    int x = (e - 1) - 8;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

/* Quantize n bf16 values (n a multiple of 32) to MXFP8: codes[n], e8m0[n / 32]. */
void ora_mx_quantize_bf16(const uint16_t *in, int n, uint8_t *codes, uint8_t *e8m0) {
    for (int b = 0; b < n / 32; b++) {
        double amax = 0;
        for (int i = 0; i < 32; i++) {
            double v = fabs((double)ora_bf16(in[32 * b + i]));
            if (v > amax) amax = v;
        }
        int x = ora_mx_exponent(amax);
        e8m0[b] = (uint8_t)(x + 127);
        for (int i = 0; i < 32; i++)
            codes[32 * b + i] = ora_e4m3_encode((double)ora_bf16(in[32 * b + i]) * ldexp(1.0, -x));
    }
}

/* Value of element i of an MXFP8 vector: E4M3 code times 2^(E8M0 byte of its block - 127). */
static REAL mx_elem(const uint8_t *codes, const uint8_t *e8m0, int i) {
    return ora_e4m3(codes[i]) * (REAL)ldexp(1.0, (int)e8m0[i / 32] - 127);
}

/* ---------------------------------------------------------------- paged addressing */

/* Blocked KV layout: a logical position maps to (block number, offset inside the block) and
 * the block number goes through the per-sequence page table ([Domestic] §3.2; [SameDay] §3.1;
 * [GPUGuide] §3.2). Returns the physical slot = physical_page * page_size + offset. */
static int64_t slot_of(const int32_t *page_table, int pages_per_seq, int page_size, int seq,
                       int64_t pos) {
    int64_t logical_page = pos / page_size;
    int64_t offset = pos % page_size;
    int64_t phys = page_table[(int64_t)seq * pages_per_seq + logical_page];
    return phys * page_size + offset;
}

/* element i of a stored vector: format 0 = bf16 bit patterns, 1 or 2 = E4M3 codes times an
 * fp32 scale (scale_row: the scale that applies to this element; ignored for bf16). */
static REAL elem(int fmt, const void *base, int64_t index, float scale_row) {
    if (fmt == 0) return ora_bf16(((const uint16_t *)base)[index]);
    return ora_e4m3(((const uint8_t *)base)[index]) * (REAL)scale_row;
}

/* ---------------------------------------------------------------- indexer scores */

/*
 * Lightweight indexer: relevance score of one history token for one query token, with
 * head-weight weighting ([CANN] §1 and §2.1; the score-then-reduce step of [Domestic] §3.1).
 * The pages do not write the formula down; this library's definition is
 *     d[h]  = sum_i q_I[h][i] * k_I[t][i]          (i ascending)
 *     s[t]  = sum_h w[h] * max(d[h], 0)            (h ascending)
 * with one k_I row per token shared by all indexer heads.
 */
static REAL score_one(int heads, int dim, const uint16_t *qrow /* [heads, dim] */,
                      const float *wrow /* [heads] */, int fmt, const void *keys,
                      const float *key_scale, int64_t slot) {
    REAL s = 0;
    float sc = key_scale ? key_scale[slot] : 1.0f;
    for (int h = 0; h < heads; h++) {
        REAL d = 0;
        for (int i = 0; i < dim; i++)
            d += ora_bf16(qrow[(int64_t)h * dim + i]) * elem(fmt, keys, slot * dim + i, sc);
        s += (REAL)wrow[h] * (d > 0 ? d : 0);
    }
    return s;
}

/*
 * The same score with the indexer in MXFP8 ([CANN] §3): the query row of each head is quantized
 * (per-group dynamic quantization, groups of 32) exactly as ora_mx_quantize_bf16 states, the
 * stored key row is MXFP8 (codes [slot, dim], E8M0 bytes [slot, dim / 32]), and the dot
 * products, ReLU and head weighting are those of score_one.
 */
static REAL score_one_mx(int heads, int dim, const uint8_t *qcodes, const uint8_t *qe8m0,
                         const float *wrow, const uint8_t *keys, const uint8_t *key_e8m0,
                         int64_t slot) {
    REAL s = 0;
    const uint8_t *kc = keys + slot * dim, *ke = key_e8m0 + slot * (dim / 32);
    for (int h = 0; h < heads; h++) {
        REAL d = 0;
        for (int i = 0; i < dim; i++)
            d += mx_elem(qcodes + (int64_t)h * dim, qe8m0 + (int64_t)h * (dim / 32), i) *
                 mx_elem(kc, ke, i);
        s += (REAL)wrow[h] * (d > 0 ? d : 0);
    }
    return s;
}

/* ora_index_scores for MXFP8 keys (see score_one_mx); dim must be a multiple of 32. */
int ora_index_scores_mx(int nq, const int32_t *q_seq, const int64_t *q_pos, int heads, int dim,
                        const uint16_t *q_idx, const float *w, const uint8_t *keys,
                        const uint8_t *key_e8m0, const int32_t *page_table, int pages_per_seq,
                        int page_size, int64_t ncols, REAL *out) {
    if (dim % 32) return 1;
    for (int r = 0; r < nq; r++)
        if (q_pos[r] >= ncols || q_pos[r] >= (int64_t)pages_per_seq * page_size) return 1;
    uint8_t *qc = malloc((size_t)nq * heads * dim);
    uint8_t *qe = malloc((size_t)nq * heads * (dim / 32));
    if (!qc || !qe) {
        free(qc);
        free(qe);
        return 1;
    }
    for (int r = 0; r < nq; r++)
        for (int h = 0; h < heads; h++)
            ora_mx_quantize_bf16(q_idx + ((int64_t)r * heads + h) * dim, dim,
                                 qc + ((int64_t)r * heads + h) * dim,
                                 qe + ((int64_t)r * heads + h) * (dim / 32));
    int64_t total = (int64_t)nq * ncols;
#pragma omp parallel for schedule(dynamic, 512)
    for (int64_t f = 0; f < total; f++) {
        int r = (int)(f / ncols);
        int64_t t = f % ncols;
        if (t > q_pos[r]) {
            out[f] = -(REAL)INFINITY;
            continue;
        }
        int64_t slot = slot_of(page_table, pages_per_seq, page_size, q_seq[r], t);
        out[f] = score_one_mx(heads, dim, qc + (int64_t)r * heads * dim,
                              qe + (int64_t)r * heads * (dim / 32), w + (int64_t)r * heads, keys,
                              key_e8m0, slot);
    }
    free(qc);
    free(qe);
    return 0;
}

/*
 * Scores of every visible position for each query row.
 *   query r belongs to sequence q_seq[r] and sits at absolute position q_pos[r]; it sees
 *   positions 0..q_pos[r] (causal, inclusive). out[r * ncols + t] = s[t] for t <= q_pos[r],
 *   -inf for q_pos[r] < t < ncols.
 *   keys: [num_pages, page_size, dim] in format key_fmt; key_scale: [num_pages, page_size].
 */
int ora_index_scores(int nq, const int32_t *q_seq, const int64_t *q_pos, int heads, int dim,
                     const uint16_t *q_idx, const float *w, int key_fmt, const void *keys,
                     const float *key_scale, const int32_t *page_table, int pages_per_seq,
                     int page_size, int64_t ncols, REAL *out) {
    for (int r = 0; r < nq; r++)
        if (q_pos[r] >= ncols || q_pos[r] >= (int64_t)pages_per_seq * page_size) return 1;
    int64_t total = (int64_t)nq * ncols;
#pragma omp parallel for schedule(dynamic, 512)
    for (int64_t f = 0; f < total; f++) {
        int r = (int)(f / ncols);
        int64_t t = f % ncols;
        if (t > q_pos[r]) {
            out[f] = -(REAL)INFINITY;
            continue;
        }
        int64_t slot = slot_of(page_table, pages_per_seq, page_size, q_seq[r], t);
        out[f] = score_one(heads, dim, q_idx + (int64_t)r * heads * dim, w + (int64_t)r * heads,
                           key_fmt, keys, key_scale, slot);
    }
    return 0;
}

/*
 * Coarse stage of hierarchical history-block selection ([SameDay] §3.1; [GPUGuide] §3.1):
 * the same score formula applied to one summary row per block that the cache already keeps,
 * so no token of an unchosen block is read. Block j of query r is visible when j * page_size <= q_pos[r];
 * its summary row is pooled[page_table[seq][j]] (bf16, [num_pages, dim]).
 * out[r * nblk_cols + j] = block score, -inf for invisible columns.
 */
int ora_block_scores(int nq, const int32_t *q_seq, const int64_t *q_pos, int heads, int dim,
                     const uint16_t *q_idx, const float *w, const uint16_t *pooled,
                     const int32_t *page_table, int pages_per_seq, int page_size,
                     int64_t nblk_cols, REAL *out) {
    int64_t total = (int64_t)nq * nblk_cols;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t f = 0; f < total; f++) {
        int r = (int)(f / nblk_cols);
        int64_t j = f % nblk_cols;
        if (j * page_size > q_pos[r] || j >= pages_per_seq) {
            out[f] = -(REAL)INFINITY;
            continue;
        }
        int64_t phys = page_table[(int64_t)q_seq[r] * pages_per_seq + j];
        out[f] = score_one(heads, dim, q_idx + (int64_t)r * heads * dim, w + (int64_t)r * heads,
                           0, pooled, NULL, phys);
    }
    return 0;
}

/* ---------------------------------------------------------------- Top-K */

typedef struct {
    REAL s;
    int64_t t;
} cand;

/* order: larger score first; equal scores (which includes -0 == +0) -> lower position first */
static int cand_cmp(const void *a, const void *b) {
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int pos_cmp(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Top-K filtering keeps the K most relevant positions and returns a discrete index set
 * ([Domestic] §3.1; [CANN] §1). Candidates are (score, position) pairs; a full sort by
 * (score desc, position asc) stands in for any selection algorithm; the first min(K, n) are
 * kept, written in ascending position order, and the row is padded with -1. */
static int topk_of(cand *c, int64_t n, int k, int32_t *out_row) {
    for (int64_t i = 0; i < n; i++)
        if (isnan((double)c[i].s)) return 1;
    qsort(c, (size_t)n, sizeof(cand), cand_cmp);
    int keep = n < k ? (int)n : k;
    for (int j = 0; j < keep; j++) out_row[j] = (int32_t)c[j].t;
    qsort(out_row, (size_t)keep, sizeof(int32_t), pos_cmp);
    for (int j = keep; j < k; j++) out_row[j] = -1;
    return 0;
}

/* Row-wise Top-K over scores[r * ncols + t] for t < n_valid[r]. */
int ora_topk(int nrows, int64_t ncols, const REAL *scores, const int64_t *n_valid, int k,
             int32_t *out) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < nrows; r++) {
        int64_t n = n_valid[r] < ncols ? n_valid[r] : ncols;
        cand *c = (cand *)malloc(sizeof(cand) * (size_t)(n > 0 ? n : 1));
        for (int64_t t = 0; t < n; t++) {
            c[t].s = scores[(int64_t)r * ncols + t];
            c[t].t = t;
        }
        bad |= topk_of(c, n, k, out + (int64_t)r * k);
        free(c);
    }
    return bad;
}

/*
 * Fine stage of the hierarchical selection ([SameDay] §3.1: token scores are computed only
 * inside the blocks the coarse stage kept): for query r the candidates are the visible tokens of the blocks
 * listed in blocks[r * nblk .. +nblk) (entries < 0 are ignored); their indexer scores are
 * computed with the token formula and the Top-K among them is returned as above.
 */
int ora_topk_in_blocks(int nq, const int32_t *q_seq, const int64_t *q_pos, int heads, int dim,
                       const uint16_t *q_idx, const float *w, int key_fmt, const void *keys,
                       const float *key_scale, const int32_t *page_table, int pages_per_seq,
                       int page_size, const int32_t *blocks, int nblk, int k, int32_t *out) {
    int bad = 0;
    for (int r = 0; r < nq; r++) {
        int64_t ncand = 0;
        for (int j = 0; j < nblk; j++) {
            int32_t b = blocks[(int64_t)r * nblk + j];
            if (b < 0) continue;
            if (b >= pages_per_seq) return 1;
            int64_t lo = (int64_t)b * page_size, hi = lo + page_size;
            if (hi > q_pos[r] + 1) hi = q_pos[r] + 1;
            if (hi > lo) ncand += hi - lo;
        }
        cand *c = (cand *)malloc(sizeof(cand) * (size_t)(ncand > 0 ? ncand : 1));
        int64_t n = 0;
        for (int j = 0; j < nblk; j++) {
            int32_t b = blocks[(int64_t)r * nblk + j];
            if (b < 0) continue;
            int64_t lo = (int64_t)b * page_size, hi = lo + page_size;
            if (hi > q_pos[r] + 1) hi = q_pos[r] + 1;
            for (int64_t t = lo; t < hi; t++) c[n++].t = t;
        }
#pragma omp parallel for schedule(dynamic, 256)
        for (int64_t i = 0; i < n; i++) {
            int64_t slot = slot_of(page_table, pages_per_seq, page_size, q_seq[r], c[i].t);
            c[i].s = score_one(heads, dim, q_idx + (int64_t)r * heads * dim,
                               w + (int64_t)r * heads, key_fmt, keys, key_scale, slot);
        }
        bad |= topk_of(c, n, k, out + (int64_t)r * k);
        free(c);
    }
    return bad;
}

/* ---------------------------------------------------------------- sparse attention */

/*
 * Sparse attention over the gathered rows of the selected positions ([CANN] §1 and §2.1:
 * the attention reads only the KV rows named by the selected indices; [Domestic] §3). For query row r, query head h (kv head g = h / (heads_q / heads_kv)):
 *     l_j = scale * sum_i q[r][h][i] * K(t_j)[g][i]      over selected t_j >= 0
 *     m   = max_j l_j
 *     o   = sum_j exp(l_j - m) * V(t_j)[g] / sum_j exp(l_j - m)
 * An empty selection gives o = 0. Element (slot, g, i) of K is k_cache[slot * k_stride +
 * g * k_head_stride + i]; likewise V. V may be the same buffer as K (a latent row whose first
 * dim_v entries are the value). fp8 rows (kv_fmt 1) are code * k_scale[slot] (v_scale[slot]).
 * kv_fmt 2 is FP8 with one scale per 128 consecutive entries within each token and head
 * ([CANN] §3: per-token-head-tile quantization with a block of 128): entry i of head g of the
 * row at slot is code * k_scale[(slot * heads_kv + g) * k_tiles + i / 128], k_tiles =
 * ceil(dim_qk / 128) (a last, shorter tile keeps its own scale); V likewise with v_tiles. A
 * latent V (the same buffer as K) passes the K scales and k_tiles, so entry i of the value is
 * scaled exactly as entry i of the key row.
 * out: [nq, heads_q, dim_v].
 */
int ora_sparse_attn(int nq, const int32_t *q_seq, const int64_t *q_pos, int heads_q,
                    int heads_kv, int dim_qk, int dim_v, const uint16_t *q, int kv_fmt,
                    const void *k_cache, const void *v_cache, const float *k_scale,
                    const float *v_scale, int64_t k_stride, int64_t v_stride,
                    int64_t k_head_stride, int64_t v_head_stride, int k_tiles, int v_tiles,
                    const int32_t *page_table, int pages_per_seq, int page_size, int k,
                    const int32_t *idx, float softmax_scale, REAL *out) {
    if (kv_fmt == 2 && (k_tiles != (dim_qk + 127) / 128 || v_tiles < (dim_v + 127) / 128)) return 1;
    if (heads_kv <= 0 || heads_q % heads_kv) return 1;
    for (int r = 0; r < nq; r++)
        for (int j = 0; j < k; j++) {
            int32_t t = idx[(int64_t)r * k + j];
            if (t > q_pos[r]) return 1;
        }
    int group = heads_q / heads_kv;
    int64_t total = (int64_t)nq * heads_q;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t f = 0; f < total; f++) {
        int r = (int)(f / heads_q), h = (int)(f % heads_q), g = h / group;
        const uint16_t *qv = q + ((int64_t)r * heads_q + h) * dim_qk;
        const int32_t *sel = idx + (int64_t)r * k;
        REAL *o = out + ((int64_t)r * heads_q + h) * dim_v;
        REAL *logit = (REAL *)malloc(sizeof(REAL) * (size_t)(k > 0 ? k : 1));
        int64_t *slots = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
        REAL m = -(REAL)INFINITY;
        int any = 0;
        for (int j = 0; j < k; j++) {
            if (sel[j] < 0) continue;
            int64_t slot = slot_of(page_table, pages_per_seq, page_size, q_seq[r], sel[j]);
            float ks = (k_scale && kv_fmt == 1) ? k_scale[slot] : 1.0f;
            REAL d = 0;
            for (int i = 0; i < dim_qk; i++) {
                if (kv_fmt == 2) ks = k_scale[(slot * heads_kv + g) * k_tiles + i / 128];
                d += ora_bf16(qv[i]) *
                     elem(kv_fmt, k_cache, slot * k_stride + g * k_head_stride + i, ks);
            }
            logit[j] = (REAL)softmax_scale * d;
            slots[j] = slot;
            if (isnan((double)logit[j])) bad = 1;
            if (logit[j] > m) m = logit[j];
            any = 1;
        }
        for (int i = 0; i < dim_v; i++) o[i] = 0;
        if (any) {
            REAL den = 0;
            for (int j = 0; j < k; j++) {
                if (sel[j] < 0) continue;
                REAL p = exp(logit[j] - m);
                float vs = (v_scale && kv_fmt == 1) ? v_scale[slots[j]] : 1.0f;
                den += p;
                for (int i = 0; i < dim_v; i++) {
                    if (kv_fmt == 2) vs = v_scale[(slots[j] * heads_kv + g) * v_tiles + i / 128];
                    o[i] += p * elem(kv_fmt, v_cache, slots[j] * v_stride + g * v_head_stride + i,
                                     vs);
                }
            }
            for (int i = 0; i < dim_v; i++) o[i] /= den;
        }
        free(logit);
        free(slots);
    }
    return bad;
}

/* ---------------------------------------------------------------- cache append */

/* Quantize one row of n bf16 values to E4M3 with one fp32 scale (the per-row format):
 * sigma = amax / 448 in fp32 (1 for an all-zero row), code = E4M3(x / sigma) with the quotient
 * rounded to fp32 first (IEEE division), then to E4M3 (nearest, ties to even, saturating). */
static float quantize_row_e4m3(const uint16_t *in, int n, uint8_t *codes) {
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float v = fabsf((float)ora_bf16(in[i]));
        if (v > amax) amax = v;
    }
    float sigma = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int i = 0; i < n; i++) {
        float y = (float)ora_bf16(in[i]) / sigma;
        codes[i] = ora_e4m3_encode((double)y);
    }
    return sigma;
}

/* bf16 of a value computed in fp64: rounded to fp32 first, then to bf16 (both to nearest even),
 * as the cache's block summaries are stored. */
static uint16_t bf16_from_f64(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf / nan unchanged */
    uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

/*
 * Cache append: the step just before the path. Each new token row r of sequence row_seq[r] at
 * position row_pos[r] is written into the paged caches at its slot (page table + offset):
 *   - indexer key: bf16 copied (idx_fmt 0), E4M3 with a row scale (1, quantize_row_e4m3), or
 *     MXFP8 (2, ora_mx_quantize_bf16) ([CANN] §3 for the FP8 formats);
 *   - KV row(s): bf16 copied (kv_fmt 0), E4M3 with a row scale over the token's whole row
 *     (1), or E4M3 with one scale per 128 entries of each head (2, [CANN] §3);
 *   - the block summary of every block that received a token, when `pooled` is given (bf16
 *     keys only): the mean of the block's valid keys (positions up to ctx_len - 1), summed in
 *     fp64 in ascending position order, divided by the count, stored as bf16_from_f64 ([SameDay]
 *     §3.1: coarse filtering reads summaries kept in the cache).
 * Either part may be absent (idx_dim 0, or heads_kv 0). A sequence of length 0 receives
 * nothing (a decode batch has one row per sequence, empty ones included). Caches are updated in
 * place.
 */
int ora_cache_append(int nrows, const int32_t *row_seq, const int64_t *row_pos,
                     const int32_t *page_table, int pages_per_seq, int page_size,
                     const int32_t *ctx_lens, int idx_dim, int idx_fmt, const uint16_t *k_idx_new,
                     void *idx_keys, float *idx_scale, uint8_t *idx_mx, uint16_t *pooled,
                     int heads_kv, int dim_qk, int dim_v, int kv_fmt, const uint16_t *k_new,
                     const uint16_t *v_new, void *k_cache, void *v_cache, float *kv_scale) {
    for (int r = 0; r < nrows; r++) {
        int b = row_seq[r];
        int64_t pos = row_pos[r];
        if (ctx_lens[b] == 0) continue; /* an empty sequence receives nothing */
        if (pos < 0 || pos >= ctx_lens[b]) return 1;
        int64_t slot = slot_of(page_table, pages_per_seq, page_size, b, pos);
        if (idx_dim > 0) {
            const uint16_t *src = k_idx_new + (int64_t)r * idx_dim;
            if (idx_fmt == 0) {
                memcpy((uint16_t *)idx_keys + slot * idx_dim, src, 2 * (size_t)idx_dim);
            } else if (idx_fmt == 1) {
                idx_scale[slot] = quantize_row_e4m3(src, idx_dim, (uint8_t *)idx_keys + slot * idx_dim);
            } else {
                ora_mx_quantize_bf16(src, idx_dim, (uint8_t *)idx_keys + slot * idx_dim,
                                     idx_mx + slot * (idx_dim / 32));
            }
        }
        if (heads_kv > 0) {
            int64_t kw = (int64_t)heads_kv * dim_qk;
            const uint16_t *src = k_new + (int64_t)r * kw;
            if (kv_fmt == 0) {
                memcpy((uint16_t *)k_cache + slot * kw, src, 2 * (size_t)kw);
                if (v_new) {
                    int64_t vw = (int64_t)heads_kv * dim_v;
                    memcpy((uint16_t *)v_cache + slot * vw, v_new + (int64_t)r * vw, 2 * (size_t)vw);
                }
            } else if (kv_fmt == 1) {
                kv_scale[slot] = quantize_row_e4m3(src, (int)kw, (uint8_t *)k_cache + slot * kw);
            } else {
                int nt = (dim_qk + 127) / 128;
                for (int g = 0; g < heads_kv; g++)
                    for (int t = 0; t < nt; t++) {
                        int n = dim_qk - 128 * t < 128 ? dim_qk - 128 * t : 128;
                        kv_scale[(slot * heads_kv + g) * nt + t] = quantize_row_e4m3(
                            src + (int64_t)g * dim_qk + 128 * t, n,
                            (uint8_t *)k_cache + slot * kw + (int64_t)g * dim_qk + 128 * t);
                    }
            }
        }
    }
    if (pooled && idx_dim > 0 && idx_fmt == 0) {
        for (int r = 0; r < nrows; r++) {
            int b = row_seq[r];
            int64_t pos = row_pos[r];
            if (ctx_lens[b] == 0) continue;
            int64_t blk = pos / page_size;
            int64_t first = blk * page_size;
            int64_t last = first + page_size - 1;
            if (last > ctx_lens[b] - 1) last = ctx_lens[b] - 1;
            int64_t phys = page_table[(int64_t)b * pages_per_seq + blk];
            for (int d = 0; d < idx_dim; d++) {
                double s = 0.0;
                for (int64_t t = first; t <= last; t++) {
                    int64_t sl = slot_of(page_table, pages_per_seq, page_size, b, t);
                    s += (double)ora_bf16(((const uint16_t *)idx_keys)[sl * idx_dim + d]);
                }
                pooled[phys * idx_dim + d] = bf16_from_f64(s / (double)(last - first + 1));
            }
        }
    }
    return 0;
}
