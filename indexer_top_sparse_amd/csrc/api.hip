// C ABI of the library: argument validation (host only, nothing is enqueued on error),
// workspace layout, launch planning and kernel launches. Declarations and the contract of
// every entry point are in include/sa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sa.h"
#include "kernels.h"

using namespace sa;

namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status st, const char *msg) {
    g_last_error = msg;
    return st;
}

sa_status hip_fail(hipError_t e, const char *where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return SA_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

// Rows of a batch and the largest row position (host side).
struct RowPlan {
    int rows = 0;
    int64_t max_pos = -1;
};

// Sequence s takes over another sequence's selection (sa_batch.reuse).
bool reuses(const sa_batch *b, int s) { return b->reuse_host && b->reuse_host[s] >= 0; }

sa_status check_batch(const sa_batch *b, RowPlan *rp) {
    if (!b) return fail(SA_ERR_INVALID, "batch is NULL");
    if (b->num_seqs < 1) return fail(SA_ERR_INVALID, "num_seqs must be >= 1");
    if (!is_pow2(b->page_size) || b->page_size > 4096)
        return fail(SA_ERR_INVALID, "page_size must be a power of two in [1, 4096]");
    if (b->pages_per_seq < 1 || b->num_pages < 1)
        return fail(SA_ERR_INVALID, "pages_per_seq and num_pages must be >= 1");
    if ((int64_t)b->num_pages * b->page_size > INT32_MAX)
        return fail(SA_ERR_UNSUPPORTED, "num_pages * page_size must fit in int32");
    if (!b->page_table || !b->ctx_lens || !b->ctx_lens_host)
        return fail(SA_ERR_INVALID, "page_table, ctx_lens and ctx_lens_host are required");
    if ((b->q_indptr == nullptr) != (b->q_indptr_host == nullptr))
        return fail(SA_ERR_INVALID, "q_indptr and q_indptr_host must both be set or both NULL");
    if ((b->reuse == nullptr) != (b->reuse_host == nullptr))
        return fail(SA_ERR_INVALID, "reuse and reuse_host must both be set or both NULL");
    if (b->reuse_host)
        for (int s = 0; s < b->num_seqs; ++s) {
            const int r = b->reuse_host[s];
            if (r < -1 || r >= s)
                return fail(SA_ERR_INVALID, "reuse[s] must be -1 or an earlier sequence");
            if (r >= 0 && (b->reuse_host[r] != -1 || b->ctx_lens_host[r] != b->ctx_lens_host[s]))
                return fail(SA_ERR_INVALID, "reuse[s] must name a sequence that selects itself, of the same length");
        }
    const int64_t cap = (int64_t)b->pages_per_seq * b->page_size;
    RowPlan p;
    for (int s = 0; s < b->num_seqs; ++s) {
        const int n = b->ctx_lens_host[s];
        if (n < 0 || n > cap) return fail(SA_ERR_INVALID, "ctx_len outside [0, pages_per_seq*page_size]");
        int ql = 1;
        if (b->q_indptr_host) {
            if (s == 0 && b->q_indptr_host[0] != 0) return fail(SA_ERR_INVALID, "q_indptr[0] != 0");
            ql = b->q_indptr_host[s + 1] - b->q_indptr_host[s];
            if (ql < 0 || ql > n) return fail(SA_ERR_INVALID, "query rows must be 0..ctx_len per sequence");
        }
        p.rows += ql;
        if (ql > 0) p.max_pos = std::max<int64_t>(p.max_pos, n - 1);
        else if (!b->q_indptr_host) p.max_pos = std::max<int64_t>(p.max_pos, n - 1);
    }
    *rp = p;
    return SA_OK;
}

sa_status check_indexer(const sa_indexer *ix) {
    if (!ix) return fail(SA_ERR_INVALID, "indexer descriptor is NULL");
    if (ix->heads < 1 || ix->heads > 64) return fail(SA_ERR_UNSUPPORTED, "indexer heads must be 1..64");
    if (ix->dim != 64 && ix->dim != 128) return fail(SA_ERR_UNSUPPORTED, "indexer dim must be 64 or 128");
    if (ix->key_dtype != SA_BF16 && ix->key_dtype != SA_FP8_E4M3 && ix->key_dtype != SA_MXFP8)
        return fail(SA_ERR_INVALID, "unknown indexer key dtype");
    if (!ix->keys || !aligned16(ix->keys)) return fail(SA_ERR_INVALID, "indexer keys NULL or not 16-byte aligned");
    if ((ix->key_dtype == SA_FP8_E4M3) != (ix->key_scale != nullptr))
        return fail(SA_ERR_INVALID, "key_scale must be given exactly for E4M3 keys");
    if ((ix->key_dtype == SA_MXFP8) != (ix->key_mx_scale != nullptr))
        return fail(SA_ERR_INVALID, "key_mx_scale must be given exactly for MXFP8 keys");
    if (ix->key_mx_scale && (reinterpret_cast<uintptr_t>(ix->key_mx_scale) & 3u))
        return fail(SA_ERR_INVALID, "key_mx_scale not 4-byte aligned");
    if (ix->pooled && !aligned16(ix->pooled)) return fail(SA_ERR_INVALID, "pooled not 16-byte aligned");
    return SA_OK;
}

sa_status check_kv(const sa_kv *kv) {
    if (!kv) return fail(SA_ERR_INVALID, "kv descriptor is NULL");
    if (kv->heads_q < 1 || kv->heads_q > 128) return fail(SA_ERR_UNSUPPORTED, "heads_q must be 1..128");
    if (kv->heads_kv != 1) return fail(SA_ERR_UNSUPPORTED, "heads_kv must be 1");
    const bool latent = kv->dim_qk == 576 && kv->dim_v == 512 && kv->v == nullptr;
    const bool small = kv->dim_qk == 128 && kv->dim_v == 128;
    if (!latent && !small) return fail(SA_ERR_UNSUPPORTED, "(dim_qk, dim_v) must be (576, 512) latent or (128, 128)");
    if (kv->dtype != SA_BF16 && kv->dtype != SA_FP8_E4M3 && kv->dtype != SA_FP8_E4M3_T128)
        return fail(SA_ERR_INVALID, "unknown kv dtype");
    if (kv->dtype != SA_BF16 && (!latent || !kv->scale))
        return fail(SA_ERR_UNSUPPORTED, "E4M3 KV needs latent rows (v == NULL) and a scale array");
    if (kv->dtype == SA_BF16 && kv->scale) return fail(SA_ERR_INVALID, "scale given for bf16 KV");
    if (!kv->k || !aligned16(kv->k) || (kv->v && !aligned16(kv->v)))
        return fail(SA_ERR_INVALID, "k/v NULL or not 16-byte aligned");
    if (!(kv->softmax_scale > 0.f) || kv->softmax_scale > 1e30f)
        return fail(SA_ERR_INVALID, "softmax_scale must be a positive finite float");
    return SA_OK;
}

int attn_splits(int rows, int k, int heads_q) {
    const int target = 256;  // workgroups: one per CU (8 waves, about 100 KB of LDS)
    const int per_split = std::max(rows, 1) * attn_hgroups(heads_q);
    int s = std::max(1, (target + per_split - 1) / per_split);
    // at least 4 tiles of 32 rows per split: below that the merge costs more than the extra
    // workgroups save
    s = std::min(s, std::max(1, (k + 127) / 128));
    // at most 2048 rows per split: the per-row slot, bias and scale tables live in LDS
    s = std::max(s, (k + kMaxSplitRows - 1) / kMaxSplitRows);
    return s;
}
int split_len(int k, int s) { return (((k + s - 1) / s) + 31) / 32 * 32; }

// Latent-row attention (bf16 rows of 576 entries, V = the first 512, up to 128 query heads).
constexpr int kAttnTarget = 256;  // workgroups that fill an MI355X (one per CU)
bool latent_shape(const sa_kv *kv) {
    return kv->dim_qk == 576 && kv->dim_v == 512 && kv->v == nullptr && kv->dtype == SA_BF16 &&
           kv->heads_q <= 128;
}
struct AttnPlan {
    bool latent;
    int tphases;  // 1: 128 heads per workgroup, 2: 64 heads per workgroup in two tile phases
    int hgroups;  // workgroups per (row, split) that divide the heads
    int splits;
    int merge;    // 1: splits merged inside the launch
    int xcd;      // 1: the workgroups of a row on one XCD
};
// Layout and splits of the latent kernel for `rows` query rows, enough workgroups to fill the
// device. When one workgroup per row would leave compute units idle and a row has more than 64
// heads, two head groups of 64 (tphases = 2) divide each row before its index set is split: the
// merge then moves half the partials. Rows of at most 64 heads always take tphases = 2 (all 8
// waves busy). Splits keep at least 4 tiles of 32 rows and at most the rows whose tables fit
// the kernel's LDS.
AttnPlan latent_plan(int rows, int k, int heads_q, int max_splits) {
    const int r = std::max(rows, 1);
    int T = 1, hg = 1;
    int s = std::max(1, (kAttnTarget + r - 1) / r);
    if (heads_q <= 64) {
        T = 2;
    } else if (s > 1) {
        T = 2;
        hg = 2;
        s = std::max(1, (kAttnTarget + 2 * r - 1) / (2 * r));
    }
    s = std::min(s, std::max(1, (k + 127) / 128));
    s = std::min(s, std::max(1, max_splits));
    const int maxrows = attn_latent_max_rows(T);
    s = std::max(s, (k + maxrows - 1) / maxrows);
    AttnPlan p{true, T, hg, s, s > 1 ? 1 : 0, hg * s > 1 ? 1 : 0};
    return p;
}

// The latent kernel's launch for `rows` query rows: a merging launch waits between the splits of
// a (row, head group), so its grid must fit `cap` resident workgroups and each group needs one
// of `row_recs` merge records. The split count drops until it fits; latent = false when no
// split count does (the other attention kernel, with a separate merge launch, runs instead).
AttnPlan latent_launch_plan(int rows, int k, int heads_q, int cap, int row_recs) {
    AttnPlan p = latent_plan(rows, k, heads_q, 1 << 30);
    auto fits = [&](const AttnPlan &q) {
        return !q.merge || (lat_grid_host(rows, q.hgroups * q.splits, q.xcd) <= cap &&
                            (int64_t)rows * q.hgroups <= row_recs);
    };
    while (!fits(p)) {
        const AttnPlan q = latent_plan(rows, k, heads_q, p.splits - 1);
        if (q.splits >= p.splits) break;
        p = q;
    }
    p.latent = fits(p);
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t err = 0, zero = 0, sync = 0, blocks = 0, idx = 0, slots = 0, part_o = 0, part_ml = 0,
           rsync = 0, total = 0;
    int row_recs = 0;  // merge records at rsync, one per (row, head group)
    int seq_recs = 0;  // selection records per stage at sync; the fused two-stage selection's
                       // token stage uses the records [seq_recs, 2 seq_recs)
};

// The regions that must hold zeros when a call starts (error word, zero row, selection and merge
// records; every launch returns its records to zero) come first, the per-call data after them.
// seq_records / row_records >= 0 size the record regions for a fixed capacity instead of this
// batch, so that they sit at the same offsets whatever the call's shapes (the fixed scratch of
// sa_decode_step_noalloc).
WsLayout ws_layout(const sa_batch *b, int rows, const sa_kv *kv, int k, int block_k,
                   int seq_records = -1, int row_records = -1) {
    WsLayout L;
    size_t off = 0;
    L.err = off;
    off += 256;
    L.zero = off;  // stays zero: source of empty gathered rows
    off += 2048;
    L.sync = off;
    const int nsr = seq_records >= 0 ? seq_records : b->num_seqs;
    L.seq_recs = nsr;
    // two stages' records when the selection is hierarchical (always with a fixed capacity, so
    // that the offsets do not depend on the call)
    const int stages = (block_k > 0 || seq_records >= 0) ? 2 : 1;
    off = align256(off + sizeof(SelSync) * (size_t)nsr * stages);
    const int rmax = std::max(rows, b->num_seqs);
    if (kv || row_records >= 0) {
        L.rsync = off;  // merge records (the groups of a merging launch fit the device)
        const int nrr = row_records >= 0 ? row_records : std::min(2 * rmax, 8192);  // (row, head group)
        L.row_recs = nrr;
        off = align256(off + sizeof(uint32_t) * kRowSyncWords * (size_t)nrr);
    }
    L.blocks = off;
    off = align256(off + sizeof(int32_t) * (size_t)b->num_seqs * (size_t)std::max(block_k, 0));
    L.idx = off;
    off = align256(off + sizeof(int32_t) * (size_t)b->num_seqs * (size_t)std::max(k, 0));
    if (kv) {
        L.slots = off;  // physical rows of the fused step's index set
        off = align256(off + sizeof(int32_t) * (size_t)b->num_seqs * (size_t)std::max(k, 0));
        // the split count only grows as rows shrink; size for the larger of the two, for
        // either kernel
        int s = std::max(attn_splits(rows, k, kv->heads_q), attn_splits(b->num_seqs, k, kv->heads_q));
        // the latent kernel's blocks cover 128 heads per (row, split) at most (head groups
        // times heads per group, rounded up to 16)
        int hq = kv->heads_q;
        if (latent_shape(kv)) {
            s = std::max(s, std::max(latent_plan(rows, k, kv->heads_q, 1 << 30).splits,
                                     latent_plan(b->num_seqs, k, kv->heads_q, 1 << 30).splits));
            hq = 128;
        }
        L.part_o = off;
        off = align256(off + sizeof(uint16_t) * (size_t)rmax * s * hq * kv->dim_v);
        L.part_ml = off;
        off = align256(off + sizeof(float) * 2 * (size_t)rmax * s * hq);
    }
    L.total = off;
    return L;
}

sa_status check_ws(void *ws, size_t bytes, size_t need) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(SA_ERR_WORKSPACE, "workspace NULL or not 256-byte aligned");
    if (bytes < need) return fail(SA_ERR_WORKSPACE, "workspace smaller than sa_workspace_size()");
    return SA_OK;
}

int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        int n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus = n;
    }
    return cus;
}

// Co-resident workgroups per CU for a kernel (cached per kernel and LDS size).
int occupancy(void *kern, int threads, size_t lds) {
    struct Entry { void *k; size_t lds; int occ; };
    static Entry cache[64];
    static int n = 0;
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
        if (cache[i].k == kern && cache[i].lds == lds) return cache[i].occ;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void *>(kern),
                                                     threads, lds) != hipSuccess)
        return -1;
    if (n < 64) cache[n++] = Entry{kern, lds, occ};
    return occ;
}

// Polls of a cross-workgroup wait: kSpinLimit, or SA_SPIN_LIMIT when set (read per call).
uint32_t spin_limit() {
    const char *e = std::getenv("SA_SPIN_LIMIT");
    if (!e || !*e) return kSpinLimit;
    char *end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    return (end && *end == 0 && v <= 0xFFFFFFFFul) ? (uint32_t)v : kSpinLimit;
}

int ncand_host(int mode, int ctx, int page_size, int block_k) {
    if (mode == 0) return ctx;
    const int nblk = (ctx + page_size - 1) / page_size;
    if (mode == 1) return nblk;
    return std::min(block_k, nblk) * page_size;
}

// The chunk of a selection launch: the smallest multiple of 64 whose workgroups (sel_groups per
// sequence, at most kMaxGroupsPerSeq each) all fit in `cap` resident workgroups, for n <= cap
// sequences with nc_of(i) candidates (< 0: a sequence that reuses another's selection, with no
// workgroups); *groups gets the launch's workgroups.
template <class F>
int plan_chunk(F nc_of, int n, int cap, int64_t *groups) {
    int nc_max = 0;
    for (int i = 0; i < n; ++i) nc_max = std::max(nc_max, nc_of(i));
    auto total_groups = [&](int c) {
        int64_t gsum = 0;
        for (int i = 0; i < n; ++i) {
            const int nc = nc_of(i);
            gsum += nc < 0 ? 0 : sel_groups(nc, c);
        }
        return gsum;
    };
    int lo = std::max(1, (nc_max + kMaxGroupsPerSeq - 1) / kMaxGroupsPerSeq);
    lo = (lo + 63) / 64;
    int hi = std::max(lo, (nc_max + 63) / 64);  // in units of 64; one workgroup per sequence fits
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        if (total_groups(64 * mid) <= cap) hi = mid;
        else lo = mid + 1;
    }
    *groups = total_groups(64 * lo);
    return 64 * lo;
}

// Launches of the fused selection for one candidate mode. All workgroups of a launch must be
// resident at once (they wait for each other), so a launch holds at most the device's resident
// capacity of workgroups; batches with more sequences than half that capacity are split into
// consecutive launches.
sa_status run_select(const sa_batch *b, const sa_indexer *ix, const void *q_idx, const float *w,
                     int mode, int k, int block_k, const int32_t *blocks, int32_t *idx_out,
                     int32_t *slots_out, uint8_t *ws, const WsLayout &L, hipStream_t st) {
    void *kern = decode_select_kernel(ix->dim, ix->heads, (int)ix->key_dtype, mode);
    if (!kern) return fail(SA_ERR_UNSUPPORTED, "no selection kernel for this key dtype and mode");
    const int threads = 512;
    const int lp = log2i(b->page_size);
    const int cus = device_cus();
    const int occ0 = occupancy(kern, threads, decode_select_dynamic_lds(mode, 64, lp));
    if (occ0 <= 0) return hip_fail(hipErrorInvalidValue, "occupancy query");
    const int per_launch = std::max(1, occ0 * cus / 2);
    for (int s0 = 0, nb = 0; s0 < b->num_seqs; s0 += nb) {
        nb = std::min(per_launch, b->num_seqs - s0);
        // capacity -> chunk -> LDS -> capacity, until the plan fits what it assumed. The chunk
        // is the smallest multiple of 64 whose workgroups (sel_groups per sequence, at most
        // kMaxGroupsPerSeq) all fit in the capacity. A chunk that does not fit (LDS, or more
        // candidates than kSelMaxChunk) halves the sequences of this
        // launch.
        int occ = occ0, chunk = 64;
        int64_t groups = 0;
        size_t lds = 0;
        for (int iter = 0;; ++iter) {
            const int cap = occ * cus;
            if (nb > cap || iter > 8) return fail(SA_ERR_UNSUPPORTED, "selection does not fit co-resident on this device");
            chunk = plan_chunk(
                [&](int i) {
                    return reuses(b, s0 + i) ? -1 : ncand_host(mode, b->ctx_lens_host[s0 + i], b->page_size, block_k);
                },
                nb, cap, &groups);
            lds = decode_select_dynamic_lds(mode, chunk, lp);
            const int o = chunk <= kSelMaxChunk ? occupancy(kern, threads, lds) : 0;
            if (o <= 0) {
                if (nb == 1) return fail(SA_ERR_UNSUPPORTED, "selection chunk exceeds the LDS of a CU");
                nb = (nb + 1) / 2;
                occ = occ0;
                iter = -1;
                continue;
            }
            if (o >= occ) break;
            occ = o;
        }
        SelectArgs a{};
        a.num_seqs = nb;
        a.lp = lp;
        a.pages_per_seq = b->pages_per_seq;
        a.heads = ix->heads;
        a.chunk = chunk;
        a.k = k;
        a.block_k = block_k;
        a.page_table = b->page_table + (int64_t)s0 * b->pages_per_seq;
        a.ctx_lens = b->ctx_lens + s0;
        a.blocks = blocks ? blocks + (int64_t)s0 * block_k : nullptr;
        a.q_idx = static_cast<const uint16_t *>(q_idx) + (int64_t)s0 * ix->heads * ix->dim;
        a.w = w + (int64_t)s0 * ix->heads;
        a.keys = static_cast<const uint8_t *>(mode == 1 ? ix->pooled : ix->keys);
        a.key_scale = ix->key_scale;
        a.key_mx = ix->key_mx_scale;
        a.idx_out = idx_out + (int64_t)s0 * k;
        a.slots_out = slots_out ? slots_out + (int64_t)s0 * k : nullptr;
        a.sync = reinterpret_cast<SelSync *>(ws + L.sync) + s0;
        a.err = reinterpret_cast<uint32_t *>(ws + L.err);
        a.spin_limit = spin_limit();
        a.reuse = b->reuse ? b->reuse + s0 : nullptr;
        if (groups == 0) continue;  // every sequence of this launch reuses another's selection
        // The grid never exceeds what the device holds at once, so every workgroup becomes
        // resident once the work queued before it has drained, and the waits between
        // workgroups of a sequence end; the waits are also spin-bounded. A plain launch is
        // used: the cooperative launch API adds a device-wide synchronisation that costs more
        // than the whole selection at small batch sizes.
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(kern, dim3((unsigned)groups), dim3(threads), args, lds, st);
        if (e != hipSuccess) return hip_fail(e, "selection launch");
    }
    return SA_OK;
}

// Both stages of the hierarchical selection in one launch (k_decode_select_2l). The token
// stage's chunk is planned as for a single-stage launch; the block stage's chunk is the
// smallest multiple of 64 that needs no more workgroups per sequence than the token stage, so
// the sequence's workgroups are the token stage's (host and kernel evaluate the same max).
// Returns SA_ERR_UNSUPPORTED (nothing enqueued) when the fused kernel does not apply.
sa_status run_select2l(const sa_batch *b, const sa_indexer *ix, const void *q_idx, const float *w,
                       int k, int block_k, int32_t *blocks, int32_t *idx_out, int32_t *slots_out,
                       uint8_t *ws, const WsLayout &L, hipStream_t st) {
    void *kern = decode_select2l_kernel(ix->dim, ix->heads, (int)ix->key_dtype);
    if (!kern) return SA_ERR_UNSUPPORTED;
    const int threads = 512;
    const int lp = log2i(b->page_size);
    const int cus = device_cus();
    auto lds_of = [&](int chunk1, int chunk2) {
        return std::max(decode_select_dynamic_lds(1, chunk1, lp), decode_select_dynamic_lds(2, chunk2, lp));
    };
    const int occ0 = occupancy(kern, threads, lds_of(64, 64));
    if (occ0 <= 0) return hip_fail(hipErrorInvalidValue, "occupancy query");
    const int per_launch = std::max(1, occ0 * cus / 2);
    for (int s0 = 0, nb = 0; s0 < b->num_seqs; s0 += nb) {
        nb = std::min(per_launch, b->num_seqs - s0);
        auto nc1 = [&](int i) { return ncand_host(1, b->ctx_lens_host[s0 + i], b->page_size, block_k); };
        auto nc2 = [&](int i) {
            return reuses(b, s0 + i) ? -1 : ncand_host(2, b->ctx_lens_host[s0 + i], b->page_size, block_k);
        };
        int occ = occ0, chunk1 = 64, chunk2 = 64;
        int64_t groups = 0;
        size_t lds = 0;
        for (int iter = 0;; ++iter) {
            const int cap = occ * cus;
            if (nb > cap || iter > 8) return SA_ERR_UNSUPPORTED;
            chunk2 = plan_chunk(nc2, nb, cap, &groups);
            int need1 = 1;  // block-stage candidates per workgroup
            for (int i = 0; i < nb; ++i) {
                if (nc2(i) < 0) continue;
                const int g2 = sel_groups(nc2(i), chunk2);
                need1 = std::max(need1, (nc1(i) + g2 - 1) / g2);
            }
            chunk1 = (need1 + 63) / 64 * 64;
            lds = lds_of(chunk1, chunk2);
            const int o = (chunk1 <= kSelMaxChunk && chunk2 <= kSelMaxChunk) ? occupancy(kern, threads, lds) : 0;
            if (o <= 0) {
                if (nb == 1) return SA_ERR_UNSUPPORTED;
                nb = (nb + 1) / 2;
                occ = occ0;
                iter = -1;
                continue;
            }
            if (o >= occ) break;
            occ = o;
        }
        SelectArgs ab{}, ac{};
        for (SelectArgs *a : {&ab, &ac}) {
            a->num_seqs = nb;
            a->lp = lp;
            a->pages_per_seq = b->pages_per_seq;
            a->heads = ix->heads;
            a->block_k = block_k;
            a->page_table = b->page_table + (int64_t)s0 * b->pages_per_seq;
            a->ctx_lens = b->ctx_lens + s0;
            a->q_idx = static_cast<const uint16_t *>(q_idx) + (int64_t)s0 * ix->heads * ix->dim;
            a->w = w + (int64_t)s0 * ix->heads;
            a->err = reinterpret_cast<uint32_t *>(ws + L.err);
            a->spin_limit = spin_limit();
            a->reuse = b->reuse ? b->reuse + s0 : nullptr;
        }
        if (groups == 0) continue;  // every sequence of this launch reuses another's selection
        ab.chunk = chunk1;
        ab.k = block_k;
        ab.keys = static_cast<const uint8_t *>(ix->pooled);
        ab.idx_out = blocks + (int64_t)s0 * block_k;
        ab.sync = reinterpret_cast<SelSync *>(ws + L.sync) + s0;
        ac.chunk = chunk2;
        ac.k = k;
        ac.keys = static_cast<const uint8_t *>(ix->keys);
        ac.key_scale = ix->key_scale;
        ac.blocks = blocks + (int64_t)s0 * block_k;
        ac.idx_out = idx_out + (int64_t)s0 * k;
        ac.slots_out = slots_out ? slots_out + (int64_t)s0 * k : nullptr;
        ac.sync = reinterpret_cast<SelSync *>(ws + L.sync) + L.seq_recs + s0;
        void *args[] = {&ab, &ac};
        hipError_t e = hipLaunchKernel(kern, dim3((unsigned)groups), dim3(threads), args, lds, st);
        if (e != hipSuccess) return hip_fail(e, "two-stage selection launch");
    }
    return SA_OK;
}

sa_status run_attn(const sa_batch *b, int rows, const sa_kv *kv, const void *q,
                   const int32_t *idx, const int32_t *slots, int k, void *out, uint8_t *ws,
                   const WsLayout &L, hipStream_t st) {
    AttnArgs a{};
    a.num_seqs = b->num_seqs;
    a.lp = log2i(b->page_size);
    a.pages_per_seq = b->pages_per_seq;
    a.heads_q = kv->heads_q;
    a.k = k;
    a.rows = rows;
    a.splits = attn_splits(rows, k, kv->heads_q);
    a.hgroups = attn_hgroups(kv->heads_q);
    a.split_len = split_len(k, a.splits);
    a.page_table = b->page_table;
    a.ctx_lens = b->ctx_lens;
    a.q_indptr = b->q_indptr;
    a.q = static_cast<const uint16_t *>(q);
    a.idx = idx;
    a.slots = slots;
    a.kc = static_cast<const uint8_t *>(kv->k);
    a.vc = static_cast<const uint8_t *>(kv->v);
    a.kv_scale = kv->scale;
    a.zero_row = ws + L.zero;
    a.scale_log2 = kv->softmax_scale * 1.4426950408889634f;
    a.out = static_cast<uint16_t *>(out);
    a.part_o = reinterpret_cast<uint16_t *>(ws + L.part_o);
    a.part_ml = reinterpret_cast<float *>(ws + L.part_ml);
    a.row_sync = reinterpret_cast<uint32_t *>(ws + L.rsync);
    a.err = reinterpret_cast<uint32_t *>(ws + L.err);
    a.spin_limit = spin_limit();
    a.merge_inside = 0;
    if (rows == 0) return SA_OK;
    if (latent_shape(kv)) {
        // the splits of a row wait for each other, so a merging grid must fit the device's
        // resident capacity (one workgroup per CU: the tile ring takes most of the LDS)
        static const int occ1 = attn_latent_occupancy(1, attn_latent_max_rows(1));
        static const int occ2 = attn_latent_occupancy(2, attn_latent_max_rows(2));
        const AttnPlan p0 = latent_plan(rows, k, kv->heads_q, 1 << 30);
        const int cap = std::max(p0.tphases == 1 ? occ1 : occ2, 0) * device_cus();
        const AttnPlan p = latent_launch_plan(rows, k, kv->heads_q, cap, L.row_recs);
        if (p.latent) {
            a.splits = p.splits;
            a.split_len = split_len(k, p.splits);
            a.merge_inside = p.merge;
            a.hgroups = p.hgroups;
            a.xcd_align = p.xcd;
            hipError_t e = launch_attn_latent(a, p.tphases, st);
            if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
            return SA_OK;
        }
    }
    hipError_t e = launch_sparse_attn(a, kv->dim_qk, kv->dim_v, kv->v != nullptr,
                                      (int)kv->dtype, st);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    return SA_OK;
}

// ------------------------------------------------------------ fixed scratch (no allocation)
// sa_decode_step_noalloc keeps its workspace in this array instead of a caller's buffer; every
// device the library runs on holds its own copy until the process ends. In host code the
// array's name is only a stand-in: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)48 << 20;
constexpr int kScratchSeqs = 64;    // sequences per call: the selection records at fixed offsets
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Hands the call's device error word to the caller (error_out may be null) and clears it.
__global__ void k_take_error(uint32_t *err, int32_t *error_out) {
    if (threadIdx.x == 0) {
        const uint32_t v = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (error_out) *error_out = (int32_t)v;
        __hip_atomic_store(err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

std::mutex g_scratch_mu;
uint8_t *g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch. The first call on a device looks it up and
// enqueues one zero fill (a kernel, not a memset) on `st`, ahead of the call's own kernels.
sa_status scratch_of_current_device(hipStream_t st, uint8_t **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "device ordinal beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        e = launch_zero(ptr, kScratchBytes, st);
        if (e != hipSuccess) return hip_fail(e, "scratch zero fill");
        g_scratch[dev] = static_cast<uint8_t *>(ptr);
    }
    *out = g_scratch[dev];
    return SA_OK;
}

}  // namespace

extern "C" {

int32_t sa_version(void) { return SA_VERSION; }

const char *sa_last_error(void) { return g_last_error.c_str(); }

const char *sa_status_string(sa_status s) {
    switch (s) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported shape or type";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t sa_workspace_size(const sa_batch *batch, const sa_kv *kv, int32_t k, int32_t block_k) {
    RowPlan rp;
    if (check_batch(batch, &rp) != SA_OK) return 0;
    return ws_layout(batch, rp.rows, kv, k, block_k).total;
}

sa_status sa_plan_selection(const int32_t *ncand, int32_t num_seqs, int32_t capacity,
                            int32_t *chunk_out, int64_t *groups_out) {
    if (!ncand || !chunk_out || !groups_out || num_seqs < 1)
        return fail(SA_ERR_INVALID, "ncand, chunk_out and groups_out are required, num_seqs >= 1");
    if (capacity < num_seqs) return fail(SA_ERR_INVALID, "capacity below one workgroup per sequence");
    for (int i = 0; i < num_seqs; ++i)
        if (ncand[i] < 0) return fail(SA_ERR_INVALID, "negative candidate count");
    int64_t groups = 0;
    *chunk_out = plan_chunk([&](int i) { return (int)ncand[i]; }, num_seqs, capacity, &groups);
    *groups_out = groups;
    return SA_OK;
}

sa_status sa_plan_latent_attention(int32_t rows, int32_t k, int32_t heads_q, int32_t capacity,
                                   int32_t row_records, int32_t *splits_out,
                                   int32_t *split_len_out, int32_t *head_groups_out,
                                   int32_t *merge_out, int32_t *grid_out) {
    if (!splits_out || !split_len_out || !head_groups_out || !merge_out || !grid_out || rows < 1 ||
        k < 1 || k > 65536 || heads_q < 1 || heads_q > 128 || capacity < 0 || row_records < 0)
        return fail(SA_ERR_INVALID, "outputs required; rows >= 1, 1 <= k <= 65536, 1 <= heads_q <= 128, "
                                    "capacity and row_records >= 0");
    const AttnPlan p = latent_launch_plan(rows, k, heads_q, capacity, row_records);
    *splits_out = p.latent ? p.splits : 0;
    *split_len_out = p.latent ? split_len(k, p.splits) : 0;
    *head_groups_out = p.latent ? p.hgroups : 0;
    *merge_out = p.latent ? p.merge : 0;
    *grid_out = p.latent ? lat_grid_host(rows, p.hgroups * p.splits, p.xcd) : 0;
    return SA_OK;
}

sa_status sa_workspace_init(void *ws, size_t bytes, void *stream) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) || bytes < 256)
        return fail(SA_ERR_WORKSPACE, "workspace NULL, misaligned or smaller than 256 bytes");
    hipError_t e = launch_zero(ws, bytes & ~(size_t)15, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "workspace zero-fill");
    return SA_OK;
}

sa_status sa_workspace_error(const void *ws, int32_t *error_host, void *stream) {
    if (!ws || !error_host) return fail(SA_ERR_INVALID, "workspace or error_host is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(error_host, ws, sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading the workspace error word");
    return SA_OK;
}

sa_status sa_index_score(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                         const float *w, float *scores, int64_t ld, void *stream) {
    RowPlan rp;
    sa_status st = check_batch(batch, &rp);
    if (st != SA_OK) return st;
    if ((st = check_indexer(ix)) != SA_OK) return st;
    if (!q_idx || !aligned16(q_idx) || !w || !scores)
        return fail(SA_ERR_INVALID, "q_idx (16-byte aligned), w and scores are required");
    if (ld < std::max<int64_t>(rp.max_pos + 1, 1)) return fail(SA_ERR_INVALID, "ld smaller than the largest row position + 1");
    if (rp.rows == 0) return SA_OK;
    ScoreArgs a;
    a.num_seqs = batch->num_seqs;
    a.lp = log2i(batch->page_size);
    a.pages_per_seq = batch->pages_per_seq;
    a.heads = ix->heads;
    a.page_table = batch->page_table;
    a.ctx_lens = batch->ctx_lens;
    a.q_indptr = batch->q_indptr;
    a.q_idx = static_cast<const uint16_t *>(q_idx);
    a.w = w;
    a.keys = static_cast<const uint8_t *>(ix->keys);
    a.key_scale = ix->key_scale;
    a.key_mx = ix->key_mx_scale;
    a.scores = scores;
    a.ld = ld;
    a.row_blocks = 0;
    if (batch->q_indptr)
        for (int b = 0; b < batch->num_seqs; ++b)
            a.row_blocks += (batch->q_indptr_host[b + 1] - batch->q_indptr_host[b] + 7) / 8;
    hipError_t e = launch_index_score(a, ix->dim, ix->heads, (int)ix->key_dtype, rp.rows, ld,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "index score launch");
    return SA_OK;
}

sa_status sa_topk(const sa_batch *batch, const float *scores, int64_t ld, int32_t k,
                  int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    RowPlan rp;
    sa_status st = check_batch(batch, &rp);
    if (st != SA_OK) return st;
    (void)ws;
    (void)ws_bytes;
    if (!scores || !idx) return fail(SA_ERR_INVALID, "scores and idx are required");
    if (k < 1 || k > 65536) return fail(SA_ERR_INVALID, "k must be in [1, 65536]");
    if (ld < 1) return fail(SA_ERR_INVALID, "ld must be >= 1");
    if (rp.rows == 0) return SA_OK;
    TopkArgs a;
    a.num_seqs = batch->num_seqs;
    a.k = k;
    a.ctx_lens = batch->ctx_lens;
    a.q_indptr = batch->q_indptr;
    a.scores = scores;
    a.ld = ld;
    a.idx = idx;
    hipError_t e = launch_topk_rows(a, rp.rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return SA_OK;
}

sa_status sa_sparse_attn(const sa_batch *batch, const sa_kv *kv, const void *q,
                         const int32_t *idx, int32_t k, void *out, void *ws, size_t ws_bytes,
                         void *stream) {
    RowPlan rp;
    sa_status st = check_batch(batch, &rp);
    if (st != SA_OK) return st;
    if ((st = check_kv(kv)) != SA_OK) return st;
    if (!q || !aligned16(q) || !idx || !out || (reinterpret_cast<uintptr_t>(out) & 7u))
        return fail(SA_ERR_INVALID, "q (16-byte aligned), idx and out (8-byte aligned) are required");
    if (k < 1 || k > 65536) return fail(SA_ERR_INVALID, "k must be in [1, 65536]");
    const WsLayout L = ws_layout(batch, rp.rows, kv, k, 0);
    if ((st = check_ws(ws, ws_bytes, L.total)) != SA_OK) return st;
    return run_attn(batch, rp.rows, kv, q, idx, nullptr, k, out, static_cast<uint8_t *>(ws), L,
                    static_cast<hipStream_t>(stream));
}

static sa_status select_impl_sources(const sa_batch *batch, const sa_indexer *ix,
                                     const void *q_idx, const float *w, int32_t k,
                                     int32_t block_k, int32_t *idx, int32_t *slots, uint8_t *wsb,
                                     const WsLayout &L, hipStream_t hs);

// The selection of every sequence: the sequences that select themselves, then (sa_batch.reuse)
// the copies to those that reuse their selection.
static sa_status select_impl(const sa_batch *batch, const RowPlan &rp, const sa_indexer *ix,
                             const void *q_idx, const float *w, int32_t k, int32_t block_k,
                             int32_t *idx, int32_t *slots, uint8_t *wsb, const WsLayout &L,
                             hipStream_t hs) {
    (void)rp;
    sa_status st = select_impl_sources(batch, ix, q_idx, w, k, block_k, idx, slots, wsb, L, hs);
    if (st != SA_OK || !batch->reuse) return st;
    hipError_t e = launch_reuse_copy(batch->reuse, batch->num_seqs, k, idx, slots, hs);
    if (e != hipSuccess) return hip_fail(e, "selection reuse copy");
    return SA_OK;
}

static sa_status select_impl_sources(const sa_batch *batch, const sa_indexer *ix,
                                     const void *q_idx, const float *w, int32_t k,
                                     int32_t block_k, int32_t *idx, int32_t *slots, uint8_t *wsb,
                                     const WsLayout &L, hipStream_t hs) {
    sa_status st;
    if (block_k > 0) {
        int32_t *blocks = reinterpret_cast<int32_t *>(wsb + L.blocks);
        // one launch for both stages when the fused kernel applies
        st = run_select2l(batch, ix, q_idx, w, k, block_k, blocks, idx, slots, wsb, L, hs);
        if (st != SA_ERR_UNSUPPORTED) return st;
        if ((st = run_select(batch, ix, q_idx, w, 1, block_k, block_k, nullptr, blocks, nullptr, wsb, L,
                             hs)) != SA_OK)
            return st;
        return run_select(batch, ix, q_idx, w, 2, k, block_k, blocks, idx, slots, wsb, L, hs);
    }
    return run_select(batch, ix, q_idx, w, 0, k, 0, nullptr, idx, slots, wsb, L, hs);
}

static sa_status check_select(const sa_batch *batch, RowPlan *rp, const sa_indexer *ix,
                              const void *q_idx, const float *w, int32_t k, int32_t block_k) {
    sa_status st = check_batch(batch, rp);
    if (st != SA_OK) return st;
    if (batch->q_indptr)
        return fail(SA_ERR_INVALID, "decode selection takes one query row per sequence (q_indptr must be NULL)");
    if ((st = check_indexer(ix)) != SA_OK) return st;
    if (!q_idx || !aligned16(q_idx) || !w) return fail(SA_ERR_INVALID, "q_idx (16-byte aligned) and w are required");
    if (k < 1 || k > 65536) return fail(SA_ERR_INVALID, "k must be in [1, 65536]");
    if (block_k < 0 || block_k > 65536) return fail(SA_ERR_INVALID, "block_k must be in [0, 65536]");
    if (block_k > 0 && ix->key_dtype != SA_BF16)
        return fail(SA_ERR_UNSUPPORTED,
                    "two-level selection needs bf16 indexer keys (its block summaries are bf16 "
                    "means of bf16 keys)");
    if (block_k > 0 && !ix->pooled) return fail(SA_ERR_INVALID, "two-level selection needs ix->pooled");
    return SA_OK;
}

sa_status sa_index_select(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                          const float *w, int32_t k, int32_t block_k, int32_t *idx_out,
                          void *ws, size_t ws_bytes, void *stream) {
    RowPlan rp;
    sa_status st = check_select(batch, &rp, ix, q_idx, w, k, block_k);
    if (st != SA_OK) return st;
    if (!idx_out) return fail(SA_ERR_INVALID, "idx_out is required");
    const WsLayout L = ws_layout(batch, rp.rows, nullptr, k, block_k);
    if ((st = check_ws(ws, ws_bytes, L.total)) != SA_OK) return st;
    return select_impl(batch, rp, ix, q_idx, w, k, block_k, idx_out, nullptr,
                       static_cast<uint8_t *>(ws),
                       L, static_cast<hipStream_t>(stream));
}

sa_status sa_block_select(const sa_batch *batch, const sa_indexer *ix, const void *q_idx,
                          const float *w, int32_t block_k, int32_t *blocks_out, void *ws,
                          size_t ws_bytes, void *stream) {
    RowPlan rp;
    if (block_k < 1) return fail(SA_ERR_INVALID, "block_k must be in [1, 65536]");
    sa_status st = check_select(batch, &rp, ix, q_idx, w, block_k, block_k);
    if (st != SA_OK) return st;
    if (!blocks_out) return fail(SA_ERR_INVALID, "blocks_out is required");
    const WsLayout L = ws_layout(batch, rp.rows, nullptr, block_k, block_k);
    if ((st = check_ws(ws, ws_bytes, L.total)) != SA_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = run_select(batch, ix, q_idx, w, 1, block_k, block_k, nullptr, blocks_out, nullptr,
                         static_cast<uint8_t *>(ws), L, hs)) != SA_OK || !batch->reuse)
        return st;
    hipError_t e = launch_reuse_copy(batch->reuse, batch->num_seqs, block_k, blocks_out, nullptr, hs);
    if (e != hipSuccess) return hip_fail(e, "selection reuse copy");
    return SA_OK;
}

sa_status sa_decode_step(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                         const void *q_idx, const float *w, const void *q, int32_t k,
                         int32_t block_k, int32_t *idx_out, void *out, void *ws,
                         size_t ws_bytes, void *stream) {
    RowPlan rp;
    sa_status st = check_select(batch, &rp, ix, q_idx, w, k, block_k);
    if (st != SA_OK) return st;
    if ((st = check_kv(kv)) != SA_OK) return st;
    if (!q || !aligned16(q) || !out || (reinterpret_cast<uintptr_t>(out) & 7u))
        return fail(SA_ERR_INVALID, "q (16-byte aligned) and out (8-byte aligned) are required");
    const WsLayout L = ws_layout(batch, rp.rows, kv, k, block_k);
    if ((st = check_ws(ws, ws_bytes, L.total)) != SA_OK) return st;
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(wsb + L.idx);
    // the selection also writes the physical rows of the index set, so the attention reads
    // them directly instead of translating positions through the page table
    int32_t *slots = reinterpret_cast<int32_t *>(wsb + L.slots);
    if ((st = select_impl(batch, rp, ix, q_idx, w, k, block_k, idx, slots, wsb, L, hs)) != SA_OK)
        return st;
    return run_attn(batch, rp.rows, kv, q, idx, slots, k, out, wsb, L, hs);
}

sa_status sa_decode_step_noalloc(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                                 const void *q_idx, const float *w, const void *q, int32_t k,
                                 int32_t block_k, int32_t *idx_out, void *out,
                                 int32_t *error_out, void *stream) {
    RowPlan rp;
    sa_status st = check_select(batch, &rp, ix, q_idx, w, k, block_k);
    if (st != SA_OK) return st;
    if ((st = check_kv(kv)) != SA_OK) return st;
    if (!q || !aligned16(q) || !out || (reinterpret_cast<uintptr_t>(out) & 7u))
        return fail(SA_ERR_INVALID, "q (16-byte aligned) and out (8-byte aligned) are required");
    if (batch->num_seqs > kScratchSeqs)
        return fail(SA_ERR_UNSUPPORTED, "sa_decode_step_noalloc: more than 64 sequences");
    // the records at fixed offsets: selection records for kScratchSeqs sequences, merge records
    // for two head groups of as many rows (decode has one row per sequence)
    const WsLayout L = ws_layout(batch, rp.rows, kv, k, block_k, kScratchSeqs, 2 * kScratchSeqs);
    if (L.total > kScratchBytes)
        return fail(SA_ERR_UNSUPPORTED, "sa_decode_step_noalloc: the call needs more than the 48 MiB scratch "
                                        "(fewer sequences or a smaller k)");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint8_t *wsb = nullptr;
    if ((st = scratch_of_current_device(hs, &wsb)) != SA_OK) return st;
    int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(wsb + L.idx);
    int32_t *slots = reinterpret_cast<int32_t *>(wsb + L.slots);
    if ((st = select_impl(batch, rp, ix, q_idx, w, k, block_k, idx, slots, wsb, L, hs)) != SA_OK)
        return st;
    if ((st = run_attn(batch, rp.rows, kv, q, idx, slots, k, out, wsb, L, hs)) != SA_OK) return st;
    hipLaunchKernelGGL(k_take_error, dim3(1), dim3(64), 0, hs, reinterpret_cast<uint32_t *>(wsb + L.err),
                       error_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "error word launch");
    return SA_OK;
}

sa_status sa_cache_append(const sa_batch *batch, const sa_indexer *ix, const sa_kv *kv,
                          const void *k_idx_new, const void *kv_new, const void *v_new,
                          void *stream) {
    RowPlan rp;
    sa_status st = check_batch(batch, &rp);
    if (st != SA_OK) return st;
    AppendArgs a{};
    a.num_seqs = batch->num_seqs;
    a.lp = log2i(batch->page_size);
    a.pages_per_seq = batch->pages_per_seq;
    a.page_table = batch->page_table;
    a.ctx_lens = batch->ctx_lens;
    a.q_indptr = batch->q_indptr;
    bool pool = false;
    if (k_idx_new) {
        if ((st = check_indexer(ix)) != SA_OK) return st;
        if (!aligned16(k_idx_new)) return fail(SA_ERR_INVALID, "k_idx_new not 16-byte aligned");
        if (ix->pooled && ix->key_dtype != SA_BF16)
            return fail(SA_ERR_UNSUPPORTED, "block summaries are kept for bf16 indexer keys only");
        a.idx_dim = ix->dim;
        a.idx_fmt = (int)ix->key_dtype;  // 0 bf16, 1 E4M3 + row scale, 2 MXFP8
        a.k_idx_new = static_cast<const uint16_t *>(k_idx_new);
        a.idx_keys = static_cast<uint8_t *>(const_cast<void *>(ix->keys));
        a.idx_scale = const_cast<float *>(ix->key_scale);
        a.idx_mx = const_cast<uint8_t *>(ix->key_mx_scale);
        a.pooled = static_cast<uint16_t *>(const_cast<void *>(ix->pooled));
        pool = ix->pooled != nullptr;
    }
    if (kv_new) {
        if ((st = check_kv(kv)) != SA_OK) return st;
        if (!aligned16(kv_new) || (v_new && !aligned16(v_new)))
            return fail(SA_ERR_INVALID, "kv_new / v_new not 16-byte aligned");
        if ((v_new != nullptr) != (kv->v != nullptr))
            return fail(SA_ERR_INVALID, "v_new must be given exactly for a separate V cache");
        a.heads_kv = kv->heads_kv;
        a.dim_qk = kv->dim_qk;
        a.dim_v = kv->dim_v;
        a.kv_fmt = kv->dtype == SA_BF16 ? 0 : (kv->dtype == SA_FP8_E4M3 ? 1 : 2);
        a.kv_new = static_cast<const uint16_t *>(kv_new);
        a.v_new = static_cast<const uint16_t *>(v_new);
        a.kc = static_cast<uint8_t *>(const_cast<void *>(kv->k));
        a.vc = static_cast<uint8_t *>(const_cast<void *>(kv->v));
        a.kv_scale = const_cast<float *>(kv->scale);
    } else if (v_new) {
        return fail(SA_ERR_INVALID, "v_new without kv_new");
    }
    if (rp.rows == 0 || (!k_idx_new && !kv_new)) return SA_OK;
    hipError_t e = launch_cache_append(a, rp.rows, pool, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cache append launch");
    return SA_OK;
}

sa_status sa_copy_pages(const sa_indexer *ix, const sa_kv *kv, int32_t page_size,
                        const int32_t *pairs, int32_t n, void *stream) {
    if (n < 0 || (n > 0 && !pairs) || page_size < 1) return fail(SA_ERR_INVALID, "pairs, n or page_size invalid");
    sa_status st;
    PageCopyArgs a{};
    a.pairs = pairs;
    const int64_t P = page_size;
    if (ix) {
        if ((st = check_indexer(ix)) != SA_OK) return st;
        const int64_t kb = ix->key_dtype == SA_BF16 ? 2 * ix->dim : ix->dim;
        a.base[0] = static_cast<uint8_t *>(const_cast<void *>(ix->keys));
        a.page_bytes[0] = P * kb;
        a.base[1] = reinterpret_cast<uint8_t *>(const_cast<float *>(ix->key_scale));
        a.page_bytes[1] = P * 4;
        a.base[2] = const_cast<uint8_t *>(ix->key_mx_scale);
        a.page_bytes[2] = P * (ix->dim / 32);
        a.base[3] = static_cast<uint8_t *>(const_cast<void *>(ix->pooled));
        a.page_bytes[3] = 2 * (int64_t)ix->dim;  // one summary row per page
    }
    if (kv) {
        if ((st = check_kv(kv)) != SA_OK) return st;
        const int64_t w = (int64_t)kv->heads_kv * kv->dim_qk;
        a.base[4] = static_cast<uint8_t *>(const_cast<void *>(kv->k));
        a.page_bytes[4] = P * (kv->dtype == SA_BF16 ? 2 * w : w);
        a.base[5] = static_cast<uint8_t *>(const_cast<void *>(kv->v));
        a.page_bytes[5] = P * 2 * (int64_t)kv->heads_kv * kv->dim_v;
        a.base[6] = reinterpret_cast<uint8_t *>(const_cast<float *>(kv->scale));
        a.page_bytes[6] = P * 4 * (kv->dtype == SA_FP8_E4M3_T128 ? (int64_t)kv->heads_kv * ((kv->dim_qk + 127) / 128) : 1);
    }
    if (n == 0) return SA_OK;
    hipError_t e = launch_copy_pages(a, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "page copy launch");
    return SA_OK;
}

size_t sa_prolog_workspace_size(const sa_prolog *p, int32_t rows) {
    if (!p || rows < 1 || p->d_model < 128 || p->d_model % 128 || p->heads < 1 || p->dim < 1) return 0;
    return prolog_workspace_bytes(rows, p->dim, p->heads, p->d_model);
}

sa_status sa_indexer_prolog(const sa_prolog *p, int32_t rows, const void *x_q, const void *x,
                            void *q_out, void *k_out, float *w_out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (!p) return fail(SA_ERR_INVALID, "prolog descriptor is NULL");
    if (rows < 1) return fail(SA_ERR_INVALID, "rows must be >= 1");
    if (p->heads < 1 || p->heads > 64) return fail(SA_ERR_UNSUPPORTED, "prolog heads must be 1..64");
    if (p->dim != 64 && p->dim != 128) return fail(SA_ERR_UNSUPPORTED, "prolog dim must be 64 or 128");
    if (p->d_q < 128 || p->d_q % 128 || p->d_model < 128 || p->d_model % 128)
        return fail(SA_ERR_UNSUPPORTED, "d_q and d_model must be positive multiples of 128");
    if (!(p->ln_eps > 0.f)) return fail(SA_ERR_INVALID, "ln_eps must be > 0");
    const void *ptrs[] = {p->w_q, p->w_k, p->w_w, x_q, x, q_out, k_out, workspace};
    for (const void *q : ptrs)
        if (!q || !aligned16(q)) return fail(SA_ERR_INVALID, "prolog buffers must be non-NULL and 16-byte aligned");
    if (!p->ln_gamma || !p->ln_beta || !w_out) return fail(SA_ERR_INVALID, "ln_gamma, ln_beta and w_out are required");
    if (workspace_bytes < prolog_workspace_bytes(rows, p->dim, p->heads, p->d_model))
        return fail(SA_ERR_WORKSPACE, "prolog workspace smaller than sa_prolog_workspace_size");
    PrologArgs a;
    a.rows = rows;
    a.heads = p->heads;
    a.dim = p->dim;
    a.d_q = p->d_q;
    a.d_model = p->d_model;
    a.x_q = static_cast<const uint16_t *>(x_q);
    a.x = static_cast<const uint16_t *>(x);
    a.w_q = static_cast<const uint16_t *>(p->w_q);
    a.w_k = static_cast<const uint16_t *>(p->w_k);
    a.w_w = static_cast<const uint16_t *>(p->w_w);
    a.gamma = p->ln_gamma;
    a.beta = p->ln_beta;
    a.eps = p->ln_eps;
    a.q_out = static_cast<uint16_t *>(q_out);
    a.w_out = w_out;
    a.k_out = static_cast<uint16_t *>(k_out);
    a.part = static_cast<float *>(workspace);
    hipError_t e = launch_prolog(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prolog launch");
    return SA_OK;
}

}  // extern "C"
