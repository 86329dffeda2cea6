// Kernel argument blocks, the per-sequence synchronisation record and the launchers that the
// C ABI (api.hip) calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Polls of a cross-workgroup wait before it expires (about a second of waiting); the
// environment variable SA_SPIN_LIMIT overrides it per call, so that tests can drive the
// failure path with every kernel still ending normally.
constexpr uint32_t kSpinLimit = 1u << 20;

constexpr int kMaxGroupsPerSeq = 512;  // workgroups sharing one sequence in a selection
constexpr int kSelMaxChunk = 32768;     // candidates of one selection workgroup (128 KiB of keys)

// Per-sequence record in the workspace used by the cross-workgroup selection. The counters, the
// failure flag and the histograms return to zero by the end of every launch, also when a wait
// expired.
constexpr int kListCap = 4096;  // threshold-bin candidates resolved through the list

struct SelSync {
    uint32_t count;   // barrier arrivals in the current launch (0 between launches)
    uint32_t left;    // workgroups past their last barrier (0 between launches)
    uint32_t fail;    // set when a wait of this launch expired (0 between launches)
    uint32_t pad[61];
    uint32_t hist[3][2048];
    uint32_t cnt[kMaxGroupsPerSeq][2];
    uint64_t list[kListCap];  // (key << 32 | ~candidate) of the threshold bin's candidates
};

// Query row -> (sequence, offset inside the sequence's rows, rows of that sequence).
__device__ __forceinline__ void row_info(const int32_t *q_indptr, int num_seqs, int row,
                                         int &seq, int &qoff, int &qlen) {
    if (!q_indptr) {
        seq = row;
        qoff = 0;
        qlen = 1;
        return;
    }
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {  // last b with q_indptr[b] <= row
        const int mid = (lo + hi + 1) >> 1;
        if (q_indptr[mid] <= row) lo = mid;
        else hi = mid - 1;
    }
    seq = lo;
    qoff = row - q_indptr[lo];
    qlen = q_indptr[lo + 1] - q_indptr[lo];
}

struct ScoreArgs {
    int num_seqs, lp, pages_per_seq, heads;
    int row_blocks;  // prefill GEMM: sum over sequences of ceil(query rows / 8)
    const int32_t *page_table, *ctx_lens, *q_indptr;
    const uint16_t *q_idx;
    const float *w;
    const uint8_t *keys;
    const float *key_scale;
    const uint8_t *key_mx;  // MXFP8 keys: E8M0 exponents [rows][dim / 32], else null
    float *scores;
    int64_t ld;
};

// Work split of the fused selection: every workgroup of a launch covers `chunk` consecutive
// candidates of one sequence (the last one of a sequence fewer); a sequence with nc candidates
// gets sel_groups(nc, chunk) workgroups. The host picks the smallest chunk (a multiple of 64)
// whose workgroups all fit on the device at once, so the longest stream per workgroup is as
// short as the device allows whatever the length mix. Host and device evaluate the same
// expression.
__host__ __device__ inline int sel_groups(int nc, int chunk) {
    return nc > 0 ? (nc + chunk - 1) / chunk : 1;
}

struct SelectArgs {
    int num_seqs, lp, pages_per_seq, heads, k, block_k;
    int chunk;  // candidates per workgroup (see sel_groups)
    const int32_t *page_table, *ctx_lens;
    const int32_t *blocks;  // [num_seqs][block_k] for the fine stage, else null
    const uint16_t *q_idx;
    const float *w;
    const uint8_t *keys;
    const float *key_scale;
    const uint8_t *key_mx;  // MXFP8 keys: E8M0 exponents [rows][dim / 32], else null
    int32_t *idx_out;    // [num_seqs][k]
    int32_t *slots_out;  // [num_seqs][k] physical rows of the selected positions, or null
    SelSync *sync;
    uint32_t *err;
    uint32_t spin_limit;  // polls of a cross-workgroup wait before it expires
    const int32_t *reuse; // [num_seqs] >= 0: the sequence reuses another's selection (no
                          // workgroups here), or null
};

struct TopkArgs {
    int num_seqs, k;
    const int32_t *ctx_lens, *q_indptr;
    const float *scores;
    int64_t ld;
    int32_t *idx;
};

// Head groups per query row: one attention workgroup per 32 query heads.
inline int attn_hgroups(int heads_q) { return (heads_q + 63) / 64; }
constexpr int kMaxSplitRows = 2048;  // selected rows per attention workgroup

struct AttnArgs {
    int num_seqs, lp, pages_per_seq, heads_q, k, splits, split_len, rows, hgroups;
    const int32_t *page_table, *ctx_lens, *q_indptr;
    const uint16_t *q;
    const int32_t *idx;
    const int32_t *slots;  // [rows][k] physical rows of idx (-1 unused), or null: translate idx
    const uint8_t *kc;  // K rows (or latent rows)
    const uint8_t *vc;  // V rows, or null when V is the head of each K row
    const float *kv_scale;
    const uint8_t *zero_row;  // >= 1152 zero bytes (source of empty staged rows)
    float scale_log2;   // softmax_scale * log2(e)
    uint16_t *out;      // bf16 [rows][heads_q][dv] (splits == 1)
    uint16_t *part_o;   // bf16 [rows][splits][heads_q][dv], normalised per split (splits > 1)
    float *part_ml;     // [rows][splits][heads_q][2]
    // latent-row kernel with the split merge inside: per (query row, head group) a record of
    // kRowSyncWords words (arrival counter, leave counter, failure flag), zero between launches
    uint32_t *row_sync;
    uint32_t *err;
    uint32_t spin_limit;  // polls of the split barrier before it expires
    int merge_inside;     // 1: the splits of a (row, head group) meet at a barrier and merge in
                          // the same launch
    int xcd_align;        // 1: the workgroups of a row get indices of one residue mod 8
};
constexpr int kRowSyncWords = 16;
// latent-row kernel (bf16 576/512 rows, up to 128 query heads); tphases 1 or 2 (128 or 64
// heads per workgroup), hgroups = head groups per row
hipError_t launch_attn_latent(const AttnArgs &a, int tphases, hipStream_t st);
int attn_latent_occupancy(int tphases, int split_len);
int attn_latent_max_rows(int tphases);  // selected rows per split (LDS tables)
int lat_grid_host(int rows, int units, int xcd_align);

// key_fmt: 0 bf16, 1 E4M3 with a row scale, 2 MXFP8 (the values of sa_dtype)
hipError_t launch_index_score(const ScoreArgs &a, int dim, int heads, int key_fmt, int rows,
                              int64_t max_cols, hipStream_t st);
void *decode_select_kernel(int dim, int heads, int key_fmt, int mode);  // null: unsupported
// both stages of the hierarchical selection in one launch, arguments (blocks stage, tokens stage)
void *decode_select2l_kernel(int dim, int heads, int key_fmt);        // null: unsupported
size_t decode_select_static_lds();
size_t decode_select_dynamic_lds(int mode, int chunk, int lp);
hipError_t launch_topk_rows(const TopkArgs &a, int rows, hipStream_t st);
// rows of sequences with reuse[s] >= 0 copied from row reuse[s] (rows of k entries; slots may
// be null)
hipError_t launch_reuse_copy(const int32_t *reuse, int num_seqs, int k, int32_t *idx,
                             int32_t *slots, hipStream_t st);
// kv_fmt: 0 bf16, 1 E4M3 with a row scale, 3 E4M3 with a scale per 128-entry tile (sa_dtype)
hipError_t launch_sparse_attn(const AttnArgs &a, int dqk, int dv, bool sep_v, int kv_fmt,
                              hipStream_t st);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

// Cache append: new token rows (the last qlen positions of each sequence) into the caches.
struct AppendArgs {
    int num_seqs, lp, pages_per_seq;
    const int32_t *page_table, *ctx_lens, *q_indptr;
    int idx_dim, idx_fmt;           // idx_fmt: 0 bf16, 1 E4M3 + row scale, 2 MXFP8
    const uint16_t *k_idx_new;      // bf16 [rows][idx_dim], or null
    uint8_t *idx_keys;
    float *idx_scale;
    uint8_t *idx_mx;
    uint16_t *pooled;               // bf16 [pages][idx_dim], or null
    int heads_kv, dim_qk, dim_v, kv_fmt;  // kv_fmt: 0 bf16, 1 E4M3 + row scale, 2 + tile scales
    const uint16_t *kv_new, *v_new;  // bf16 [rows][heads_kv][dim_qk] / [dim_v], or null
    uint8_t *kc, *vc;
    float *kv_scale;
};
hipError_t launch_cache_append(const AppendArgs &a, int rows, bool pool, hipStream_t st);

// Whole-page copies across the cache tables: page src of every table to page dst.
constexpr int kPageTables = 7;  // keys, key scales, MXFP8 exponents, summaries, K, V, KV scales
struct PageCopyArgs {
    const int32_t *pairs;               // device [n][2] (src, dst)
    uint8_t *base[kPageTables];         // table base, or null
    int64_t page_bytes[kPageTables];    // bytes of one page in the table
};
hipError_t launch_copy_pages(const PageCopyArgs &a, int n, hipStream_t st);

// Indexer prolog: query / key / head-weight projections of new token rows, then the key's
// LayerNorm.
struct PrologArgs {
    int rows, heads, dim, d_q, d_model;
    const uint16_t *x_q, *x;         // bf16 [rows][d_q], [rows][d_model]
    const uint16_t *w_q, *w_k, *w_w;  // bf16 [heads*dim][d_q], [dim][d_model], [heads][d_model]
    const float *gamma, *beta;       // fp32 [dim]
    float eps;
    uint16_t *q_out;                 // bf16 [rows][heads][dim]
    float *w_out;                    // fp32 [rows][heads]
    uint16_t *k_out;                 // bf16 [rows][dim]
    float *part;                     // fp32 [slices][rows][dim + heads] partial sums (workspace)
};
hipError_t launch_prolog(const PrologArgs &a, hipStream_t st);
size_t prolog_workspace_bytes(int rows, int dim, int heads, int d_model);

}  // namespace sa
