/*
 * sa.h -- C ABI of the index-selected sparse attention library for AMD MI355X (gfx950).
 *
 * The path: a lightweight indexer scores every visible history token of a query, Top-K keeps
 * the K most relevant positions, and attention runs only over the key/value rows of those
 * positions, read from a paged (blocked) KV cache.
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
 * Conventions shared by every entry point
 *  - Pointers marked "device" are HIP device allocations; "host" pointers are read during the
 *    call only. The caller owns every buffer; the library allocates no device memory.
 *  - All work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and is
 *    asynchronous: no entry point synchronizes the host with the device.
 *  - Host-detectable errors (NULL pointers, sizes out of range, unsupported combinations, a
 *    too-small workspace) return SA_ERR_INVALID / SA_ERR_UNSUPPORTED / SA_ERR_WORKSPACE and
 *    enqueue nothing. A failed launch returns SA_ERR_HIP; sa_last_error() then holds the
 *    message. Device-side contents (page ids, positions, lengths) are trusted: the host copies
 *    of the context lengths must equal the device copies, page ids must be < num_pages and
 *    selected positions must be visible to their query (see each call).
 *  - Positions are logical token positions (int32) inside a sequence, never physical slots,
 *    so an index set stays valid when pages move; the consumer translates position t to
 *    slot page_table[seq][t / page_size] * page_size + t % page_size ([Domestic] §3.2:
 *    block number plus in-block offset; [GPUGuide] §3.1: index format aligned with the
 *    attention consumer).
 *  - Query rows: sequence b owns rows q_indptr[b] .. q_indptr[b+1]-1, which are its last
 *    q_len_b tokens (appended causally); row j of b sits at position
 *    ctx_len_b - q_len_b + (j - q_indptr[b]) and sees positions 0..that position inclusive.
 *    With q_indptr == NULL every sequence has exactly one row (decode) at ctx_len_b - 1.
 *  - Re-entrancy: the library's only state is a per-thread error message, per-kernel launch
 *    settings, and the per-device scratch of sa_decode_step_noalloc. Calls from several host
 *    threads are safe; calls sharing one workspace (or the scratch) must be ordered on one
 *    stream.
 *  - Co-residency: the fused selection (sa_index_select, sa_block_select, sa_decode_step) and
 *    the latent-row attention with its split merge (bf16 576/512 rows in sa_sparse_attn and
 *    sa_decode_step) have workgroups of one launch wait for each other. The host sizes those
 *    grids to what the device holds at once, assuming the launch has the device to itself;
 *    kernels running at the same time (other streams, other processes) can hold compute units
 *    and keep some workgroups from starting. Every such wait is bounded (2^20 polls, about a
 *    second; the environment variable SA_SPIN_LIMIT, read per call, overrides the count). When
 *    one expires, the call still ends with a defined result: every sequence whose selection
 *    waited too long gets index -1 in every slot (and so output 0), every group of a row's
 *    heads whose split barrier expired (the latent attention merges 64 or 128 heads of a row
 *    together) gets output 0, and bit 0 of the workspace error word is set
 *    (sa_workspace_error). The workspace is left ready for the next call.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_VERSION 1

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID = 1,     /* an argument violates a precondition; nothing enqueued */
    SA_ERR_UNSUPPORTED = 2, /* valid, but no kernel exists for this shape/type; nothing enqueued */
    SA_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned or smaller than required */
    SA_ERR_HIP = 4          /* a HIP runtime call failed; see sa_last_error() */
} sa_status;

typedef enum sa_dtype {
    SA_BF16 = 0,     /* bfloat16 */
    SA_FP8_E4M3 = 1, /* OCP E4M3 codes (max 448) times one fp32 scale per stored row */
    SA_MXFP8 = 2,    /* OCP microscaling: E4M3 codes, and for every 32 consecutive entries of a
                        row one E8M0 byte e giving the scale 2^(e - 127) (indexer keys only) */
    SA_FP8_E4M3_T128 = 3 /* OCP E4M3 codes times one fp32 scale per 128 consecutive entries of a
                            row, a shorter last tile keeping its own (KV only) */
} sa_dtype;

/* Sequences, their lengths and the page table of the blocked KV layout ([Domestic] §3.2;
 * [SameDay] §3.1 and §3.2: fixed-size blocks directly indexable by the selection; [GPUGuide]
 * §3.2: block location metadata). */
typedef struct sa_batch {
    int32_t num_seqs;             /* >= 1 */
    int32_t page_size;            /* tokens per page: a power of two, 1..4096 */
    int32_t pages_per_seq;        /* row stride of page_table; ctx_len <= pages_per_seq*page_size */
    int32_t num_pages;            /* physical pages held by every cache passed with this batch */
    const int32_t *page_table;    /* device [num_seqs][pages_per_seq]: logical -> physical page */
    const int32_t *ctx_lens;      /* device [num_seqs]: tokens in each sequence (>= 0) */
    const int32_t *ctx_lens_host; /* host   [num_seqs]: the same values (planning, validation) */
    const int32_t *q_indptr;      /* device [num_seqs+1] query-row offsets, or NULL (decode) */
    const int32_t *q_indptr_host; /* host copy of q_indptr; NULL exactly when q_indptr is NULL */
    /* Selection reuse for requests that share a history ([SameDay] §3.1: requests sharing a
     * history prefix can reuse selection results). NULL, or device [num_seqs] with a host copy:
     * reuse[s] = -1, or the index of an earlier sequence whose index set sequence s takes over.
     * The caller guarantees what makes the two selections equal: the same context length, the
     * same key cache contents at every position (typically the same pages), and the same
     * indexer query row and head weights. The fused selection (sa_index_select,
     * sa_block_select, sa_decode_step, sa_decode_step_noalloc) then scores and selects only
     * the other sequences and copies the index sets (and, in the fused step, the physical rows)
     * to the reusing ones; the attention still runs for every sequence. Other entry points
     * ignore it. Host-checked: -1 <= reuse[s] < s, reuse[reuse[s]] = -1, equal lengths. */
    const int32_t *reuse;
    const int32_t *reuse_host;
} sa_batch;

/* The lightweight indexer's cache ([CANN] §1 and §2.1). One key row of `dim` entries per token,
 * shared by all indexer heads. Score of position t for a query row with indexer queries
 * q_I[heads][dim] and head weights w[heads] (fp32 accumulation):
 *     s[t] = sum_h w[h] * max(q_I[h] . k_I[t], 0)
 * (relevance scoring with head-weight weighting; the pages leave the formula open and this
 * library fixes it as written). For E4M3 keys, k_I[t] = code * key_scale[t].
 *
 * MXFP8 keys: the indexer runs in MXFP8 with per-group dynamic quantization and groups of 32
 * ([CANN] §3). Entry i of a stored key row is code[i] * 2^(key_mx_scale[i / 32] - 127), and the
 * library quantizes each head's bf16 query row the same way before the dot products: for every
 * 32 consecutive entries, X = floor(log2(max |v|)) - 8 clamped to [-127, 127] (-127 when all are
 * zero), code = E4M3(v / 2^X) rounded to nearest with ties to even and saturated at +-448. The
 * dot products then use the decoded values (fp32 accumulation).
 *
 * Two-level selection (block_k > 0) needs bf16 keys: its block summaries are bf16 means of the
 * block's bf16 keys, which an E4M3 or MXFP8 cache no longer holds; with other key types the
 * calls return SA_ERR_UNSUPPORTED. */
typedef struct sa_indexer {
    int32_t heads;            /* H_I: 1..64 */
    int32_t dim;              /* d_I: 64 or 128 */
    sa_dtype key_dtype;       /* SA_BF16, SA_FP8_E4M3 or SA_MXFP8 */
    const void *keys;         /* device [num_pages][page_size][dim] */
    const float *key_scale;   /* device [num_pages][page_size] for E4M3 keys, else NULL */
    const void *pooled;       /* device bf16 [num_pages][dim]: one summary key per page for
                                 two-level selection ([SameDay] §3.1: coarse filtering over
                                 summaries already held in the cache), or NULL */
    const uint8_t *key_mx_scale; /* device [num_pages][page_size][dim / 32] E8M0 bytes for
                                    SA_MXFP8 keys (4-byte aligned), else NULL */
} sa_indexer;

/* The attention KV cache. One KV head (MQA/MLA style: every query head reads the same row).
 * Row of slot s: K = k[s][0..dim_qk), V = v[s][0..dim_v), or, when v == NULL, V is the first
 * dim_v entries of the K row (a latent row as in MLA). For E4M3 rows, value = code *
 * scale[s] (one scale per row, used for K and V). For E4M3 rows with 128-entry tiles ([CANN] §3:
 * FP8 KV quantized per token-head-tile with a block of 128), entry i of the row at slot s is
 * code * scale[s * 5 + i / 128]: five scales per 576-entry latent row, the fifth for the 64
 * entries 512..575; entry i < 512 of V uses the scale of entry i of the row. */
typedef struct sa_kv {
    int32_t heads_q;          /* query heads: 1..128 */
    int32_t heads_kv;         /* must be 1 */
    int32_t dim_qk;           /* 576 (latent, v == NULL, dim_v 512) or 128 (dim_v 128) */
    int32_t dim_v;            /* 512 or 128 */
    sa_dtype dtype;           /* SA_BF16, SA_FP8_E4M3 or SA_FP8_E4M3_T128 (E4M3 only with
                                 v == NULL) */
    const void *k;            /* device [num_pages][page_size][dim_qk] */
    const void *v;            /* device [num_pages][page_size][dim_v], or NULL (latent) */
    const float *scale;       /* device [num_pages][page_size] for E4M3, [num_pages][page_size][5]
                                 for E4M3 with 128-entry tiles, else NULL */
    float softmax_scale;      /* logits are softmax_scale * (q . K) */
} sa_kv;

/*
 * sa_index_score -- indexer scores of every visible position, written to HBM (used by Prefill
 * and by tests; the fused decode path never writes scores). "Scoring -- reduction" of
 * [Domestic] §3.1; [CANN] §2.1.
 *   q_idx  device bf16 [rows][heads][dim]   (rows = num_seqs, or q_indptr_host[num_seqs])
 *   w      device fp32 [rows][heads]
 *   scores device fp32 [rows][ld]: column t holds s[t] for t <= the row's position and -inf
 *          for the remaining columns; ld >= (largest row position) + 1.
 */
sa_status sa_index_score(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                         const float *w, float *scores, int64_t ld, void *stream);

/*
 * sa_topk -- Top-K filtering ([Domestic] §3.1; [CANN] §1): for each query row, the k largest
 * of scores[row][0 .. position] ordered by (score descending, position ascending; -0 equals
 * +0), written in ascending position order and padded with -1 when fewer than k positions are
 * visible. Radix selection, no sort. Scores must not be NaN.
 *   scores device fp32 [rows][ld];  idx device int32 [rows][k];  1 <= k <= 65536.
 */
sa_status sa_topk(const sa_batch *batch, const float *scores, int64_t ld, int32_t k,
                  int32_t *idx, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_sparse_attn -- attention of each query row over the rows of its selected positions only
 * ([CANN] §1 and §2.1: the attention reads only the KV rows that the index set names;
 * [Domestic] §3). For query head g: logits softmax_scale * q[g] . K(t) over the
 * selected t, softmax in fp32, o[g] = sum p * V(t) / sum p; an empty selection gives 0.
 *   q   device bf16 [rows][heads_q][dim_qk]
 *   idx device int32 [rows][k]: positions in any order, -1 = unused; every other entry must
 *       be visible to its row (not checked on the device).
 *   out device bf16 [rows][heads_q][dim_v]
 */
sa_status sa_sparse_attn(const sa_batch *batch, const sa_kv *kv, const void *q,
                         const int32_t *idx, int32_t k, void *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * sa_index_select -- the lightweight indexer as one composite Decode operator ([CANN] §2.1:
 * relevance scoring, head-weight weighting and Top-K fused, reading the paged cache directly;
 * [CANN] §2.2: the indexer returns top-k indices). One query row per sequence
 * (batch->q_indptr must be NULL). Scores are never written to HBM: each workgroup keeps its
 * chunk of a sequence's scores in LDS, and an exact radix selection runs across the
 * workgroups that share the sequence. Hierarchical selection when block_k > 0 as described
 * for sa_decode_step.
 *   q_idx device bf16 [num_seqs][ix->heads][ix->dim];  w device fp32 [num_seqs][ix->heads]
 *   idx_out device int32 [num_seqs][k]: selected positions, ascending, -1 padded
 */
sa_status sa_index_select(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                          const float *w, int32_t k, int32_t block_k, int32_t *idx_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_block_select -- the coarse stage of hierarchical selection on its own ([SameDay] §3.1:
 * candidate blocks are shortlisted from summaries the cache already holds; [GPUGuide] §3.1).
 * Block j (= logical page j) of sequence b is scored with the indexer formula on its summary
 * row ix->pooled[page_table[b][j]]; the block_k best visible blocks are kept (ties -> lower
 * block). This is the first launch of the hierarchical path of sa_index_select and
 * sa_decode_step. One query row per sequence (batch->q_indptr must be NULL).
 *   q_idx device bf16 [num_seqs][ix->heads][ix->dim];  w device fp32 [num_seqs][ix->heads]
 *   blocks_out device int32 [num_seqs][block_k]: kept logical block numbers, ascending,
 *       -1 padded when a sequence has fewer than block_k blocks;  1 <= block_k <= 65536.
 */
sa_status sa_block_select(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                          const float *w, int32_t block_k, int32_t *blocks_out,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_decode_step -- the fused Decode path: sa_index_select followed by sa_sparse_attn on the
 * same stream, with the index set kept in the workspace ([GPUGuide] §3.3: decode fuses index
 * selection with attention to cut launches; [GPUGuide] §3.1 and [CANN] §2: no score
 * write-back). One query row per sequence (batch->q_indptr must be NULL).
 * With block_k > 0, selection is hierarchical ([SameDay] §3.1; [GPUGuide] §3.1): blocks
 * (= pages) are scored from ix->pooled, the block_k best blocks are kept (ties -> lower
 * block), and the token Top-K is taken among the visible tokens of the kept blocks.
 *   q_idx device bf16 [num_seqs][ix->heads][ix->dim];  w device fp32 [num_seqs][ix->heads]
 *   q     device bf16 [num_seqs][kv->heads_q][kv->dim_qk]
 *   idx_out device int32 [num_seqs][k] (selected positions, ascending, -1 padded) or NULL
 *   out   device bf16 [num_seqs][kv->heads_q][kv->dim_v]
 */
sa_status sa_decode_step(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                         const void *q_idx, const float *w, const void *q, int32_t k,
                         int32_t block_k, int32_t *idx_out, void *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * sa_decode_step_noalloc -- sa_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results, with the workspace taken from a fixed scratch array inside the library
 * instead of a caller's buffer. Neither this call nor the kernels it launches allocate (no
 * hipMalloc, hipFree or allocating library routine).
 *  - Scratch: 48 MiB of device memory on every device the library runs on (a file-scope device
 *    array), held until the process ends. Limits: num_seqs <= 64, and the call's workspace,
 *    laid out with its records sized for 64 sequences, must fit in 48 MiB (with k = 2048 and
 *    128 query heads over 576/512 latent rows, every batch of up to 64 sequences does). A
 *    larger call returns SA_ERR_UNSUPPORTED and enqueues nothing.
 *  - Every call on a device shares that device's scratch, which keeps the last call's contents:
 *    calls that overlap on one device (on different streams, or from threads without ordering
 *    between them) race, and their results are undefined. Order them on one stream.
 *  - The first call on a device (the caller's current device, which must be the stream's) looks
 *    the scratch up and enqueues one zero fill of it on `stream` (a kernel, no memset).
 *  - error_out: device int32, or NULL. Once the call's kernels are done it receives the call's
 *    device error word (as sa_workspace_error reports it for a workspace), which is then
 *    cleared for the next call.
 * Other arguments as sa_decode_step.
 */
sa_status sa_decode_step_noalloc(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                                 const void *q_idx, const float *w, const void *q, int32_t k,
                                 int32_t block_k, int32_t *idx_out, void *out,
                                 int32_t *error_out, void *stream);

/*
 * sa_cache_append -- the cache writes of the step just before the path: every new token's
 * indexer key and KV row go into the paged caches at their slots, quantized into the caches'
 * formats, and the summary of every block that received a token is recomputed ([SameDay] §3.1:
 * coarse filtering reads block summaries the cache keeps; [CANN] §3: the FP8 formats).
 * New tokens: with batch->q_indptr == NULL one per sequence, at position ctx_lens[b] - 1;
 * otherwise rows q_indptr[b] .. q_indptr[b+1]-1 of sequence b, at positions ctx_lens[b] - n_b ..
 * ctx_lens[b] - 1 (n_b its row count). The lengths already count the new tokens, and their pages
 * must be mapped in the page table. Sequences of length 0 receive nothing.
 *   k_idx_new device bf16 [rows][ix->dim], or NULL to leave the indexer cache unchanged (ix may
 *             then be NULL)
 *   kv_new    device bf16 [rows][kv->heads_kv][kv->dim_qk], or NULL to leave the KV cache
 *             unchanged (kv may then be NULL)
 *   v_new     device bf16 [rows][kv->heads_kv][kv->dim_v] exactly when kv->v is a separate cache
 * Written through the descriptors' pointers: ix->keys, ix->key_scale / ix->key_mx_scale,
 * ix->pooled (bf16 keys only), kv->k, kv->scale, kv->v.
 *   E4M3 (row or 128-entry tile): sigma = group max |x| / 448 in fp32 (1 for all zeros), code =
 *     E4M3(x / sigma), the quotient an IEEE fp32 division, rounded to nearest even, saturating.
 *   MXFP8: as described for sa_indexer.
 *   Block summary: mean of the block's keys at positions <= ctx_lens[b] - 1, summed in fp64 in
 *     position order, divided by their count, rounded to fp32 and then to bf16.
 * Errors: SA_ERR_INVALID for NULL or misaligned buffers, or lengths shorter than the new rows;
 * SA_ERR_UNSUPPORTED for summaries over non-bf16 keys.
 */
sa_status sa_cache_append(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                          const void *k_idx_new, const void *kv_new, const void *v_new,
                          void *stream);

/*
 * Paged cache allocator (host side; [SameDay] §3.1: fixed-size blocks that the sparse selection
 * indexes directly, reference counts and copy-on-write for requests sharing a prefix; §3.2:
 * blocks acquired incrementally during decoding and reclaimed once no request references them;
 * §4.3: coalescing and splitting of free blocks, an emergency reserve). The pool only hands out
 * page numbers; it owns no device memory. Its page tables feed sa_batch. Calls on one pool are
 * serialised by a lock.
 *   Free pages form runs of consecutive pages; a freed page merges with the runs it touches, and
 *   an allocation splits a run. A sequence growing by n pages takes the page right after its
 *   last one when free, else the smallest run holding all n, else pages from the largest runs.
 *   The last emergency_pages free pages go only to urgent requests.
 */
typedef struct sa_pool sa_pool;
/* NULL for num_pages < 1, page_size < 1 or emergency_pages outside [0, num_pages] */
sa_pool *sa_pool_create(int32_t num_pages, int32_t page_size, int32_t emergency_pages);
void sa_pool_destroy(sa_pool *pool);
/* free pages, number of free runs, longest free run (any pointer may be NULL) */
sa_status sa_pool_stats(sa_pool *pool, int32_t *free_pages, int32_t *free_runs, int32_t *largest_run);
/* sequences hold pages that a page count references; -1 on error */
int32_t sa_seq_new(sa_pool *pool);
/* a new sequence sharing every page (and the length) of `parent`: a shared prefix */
int32_t sa_seq_fork(sa_pool *pool, int32_t parent);
/* Grows `seq` to new_len tokens, taking pages on demand. When the page that receives the first
 * new token is shared with another sequence it is replaced by a fresh page (copy-on-write): the
 * (old, new) page pair is written to copies[0..1] and *n_copies = 1, and the caller copies the
 * page's contents (sa_copy_pages) before writing the new token. urgent != 0 may use the
 * emergency reserve. SA_ERR_WORKSPACE when the pool cannot supply the pages (nothing changes);
 * max_copies must be >= 1 when a copy can arise. new_len <= the current length does nothing. */
sa_status sa_seq_reserve(sa_pool *pool, int32_t seq, int32_t new_len, int32_t urgent,
                         int32_t *copies, int32_t max_copies, int32_t *n_copies);
/* Releases `seq`: each of its pages loses one reference; unreferenced pages are free again. */
sa_status sa_seq_free(sa_pool *pool, int32_t seq);
int32_t sa_seq_len(sa_pool *pool, int32_t seq);
/* Physical page of each logical page of `seq` (*n_pages of them); SA_ERR_WORKSPACE when more
 * than max_pages. */
sa_status sa_seq_page_table(sa_pool *pool, int32_t seq, int32_t *page_table, int32_t max_pages,
                            int32_t *n_pages);
int32_t sa_pool_refcount(sa_pool *pool, int32_t page);

/* Device copies of whole pages in every cache table the descriptors name (indexer keys and
 * their scales, block summaries, K, V and their scales): for each pair i, page pairs[2i] to
 * page pairs[2i+1] (device int32 [n][2]), e.g. the copy-on-write pairs of sa_seq_reserve.
 * ix or kv may be NULL. Pairs must name distinct destinations. */
sa_status sa_copy_pages(const sa_indexer *ix, const sa_kv *kv, int32_t page_size,
                        const int32_t *pairs, int32_t n, void *stream);

/* Weights of the indexer prolog (synthetic in this library's workloads; no trained weights are
 * involved). Weights are [out_features][in_features], row-major bf16. */
typedef struct sa_prolog {
    int32_t heads;           /* H_I: 1..64 */
    int32_t dim;             /* d_I: 64 or 128 */
    int32_t d_q;             /* width of the query input: a positive multiple of 128 */
    int32_t d_model;         /* width of the hidden input: a positive multiple of 128 */
    const void *w_q;         /* device bf16 [heads * dim][d_q] */
    const void *w_k;         /* device bf16 [dim][d_model] */
    const void *w_w;         /* device bf16 [heads][d_model] */
    const float *ln_gamma;   /* device fp32 [dim] */
    const float *ln_beta;    /* device fp32 [dim] */
    float ln_eps;            /* > 0 */
} sa_prolog;

/*
 * sa_indexer_prolog -- the input preparation of the indexer for `rows` new tokens ([CANN]
 * §2.2: Q projection and K normalization, Q quantization and the head-weight projection, as
 * independent work ahead of the indexer):
 *     q_I[r][h][:] = x_q[r] . W_q[h*dim .. h*dim + dim - 1]^T        (bf16 out, fp32 sums)
 *     k_I[r]       = LayerNorm(x[r] . W_k^T) * gamma + beta           (bf16 out)
 *     w[r][h]      = x[r] . W_w[h]^T                                   (fp32 out)
 * LayerNorm: mean and biased variance over the dim entries, (y - mean) / sqrt(var + eps).
 * q_I and w feed the indexer (an MXFP8 indexer quantizes q_I itself), k_I is the new token's
 * indexer key for sa_cache_append. The three projections run in one launch, the LayerNorm in a
 * second one, on `stream`.
 *   x_q device bf16 [rows][d_q];  x device bf16 [rows][d_model]
 *   q_out device bf16 [rows][heads][dim];  k_out device bf16 [rows][dim];  w_out fp32 [rows][heads]
 *   workspace: device, >= sa_prolog_workspace_size(p, rows) bytes, 16-byte aligned (partial
 *              sums of the key and head-weight projections)
 * Errors: SA_ERR_INVALID for NULL or misaligned pointers, rows < 1 or a small workspace;
 * SA_ERR_UNSUPPORTED for other shapes.
 */
sa_status sa_indexer_prolog(const sa_prolog *p, int32_t rows, const void *x_q, const void *x,
                            void *q_out, void *k_out, float *w_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace bytes of sa_indexer_prolog for `rows` tokens (0 for an invalid descriptor):
 * 4 * rows * (dim + heads) * (d_model / s), s = 512, 256 or 128, the largest dividing d_model. */
size_t sa_prolog_workspace_size(const sa_prolog *p, int32_t rows);

/* Workspace bytes that every entry point above needs for this batch, cache shape, k and
 * block_k (kv may be NULL when only indexer/Top-K calls use the workspace). */
size_t sa_workspace_size(const sa_batch *batch, const sa_kv *kv, int32_t k, int32_t block_k);

/* Zero-fills a workspace on `stream` (with a kernel). Required once before the first use of a
 * workspace; every call that completes leaves the workspace ready for the next one. */
sa_status sa_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Synchronizes `stream` and reads the workspace's device error word: 0 = no device-side
 * failure, otherwise a bitmask (1 = a cross-workgroup wait exceeded its spin limit; the
 * affected results are the defined failure results described under co-residency above). The
 * word is sticky: it keeps its bits until the workspace is initialised again. */
sa_status sa_workspace_error(const void *workspace, int32_t *error_host, void *stream);

/*
 * Launch planning, host only (no device call): the capacity arithmetic that the calls above
 * use to size grids whose workgroups wait for each other, exposed for inspection and tests.
 *
 * sa_plan_selection -- one launch of the fused selection. Sequence s has ncand[s] candidates
 * (its visible tokens, blocks, or kept-block tokens); `capacity` is the number of selection
 * workgroups the device holds at once (workgroups per CU x CUs). Writes the chunk (candidates
 * per workgroup: the smallest multiple of 64 for which every sequence needs at most 512
 * workgroups, ceil(ncand / chunk) or 1 when empty, and all of them together fit in `capacity`)
 * and the launch's workgroup count. SA_ERR_INVALID for NULL pointers, num_seqs < 1, a
 * negative count or capacity < num_seqs.
 */
sa_status sa_plan_selection(const int32_t *ncand, int32_t num_seqs, int32_t capacity,
                            int32_t *chunk_out, int64_t *groups_out);

/*
 * sa_plan_latent_attention -- the latent-row attention launch (bf16 576/512 rows) for `rows`
 * query rows of k selected rows each and heads_q query heads: splits per (row, head group),
 * split length (a multiple of 32, at most 2048 rows, or 1024 with two head groups), head
 * groups per row (1, or 2 of 64 heads when a row has more than 64 heads and one workgroup per
 * row would leave the device partly idle), merge (1: the splits of a (row, head group) merge
 * inside the launch) and grid. A merging launch must fit `capacity` resident workgroups and
 * needs one of `row_records` merge records per (row, head group); when no split count allows
 * that, splits = 0 (the other attention kernel, with a separate merge launch, runs).
 */
sa_status sa_plan_latent_attention(int32_t rows, int32_t k, int32_t heads_q, int32_t capacity,
                                   int32_t row_records, int32_t *splits_out,
                                   int32_t *split_len_out, int32_t *head_groups_out,
                                   int32_t *merge_out, int32_t *grid_out);

const char *sa_status_string(sa_status status);
const char *sa_last_error(void); /* message of the last SA_ERR_HIP on this thread */
int32_t sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
