// Lightweight indexer on gfx950: page-table-driven key stream, 64-head dot products on
// MFMA, ReLU + head-weighted reduction in registers, and (decode) an exact radix Top-K across
// the workgroups of a sequence with the scores kept in LDS.
//
// Pages cited: "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on
// Huawei Ascend CANN Architecture" (CANN) §1, §2.1; "Engineering Path for Day-0 Adaptation of
// Trillion-Scale Sparse Models on Domestic AI Accelerators" (Domestic) §3.1-§3.3; "How the
// Ascend Computing Platform Achieves Same-Day Inference Adaptation for Ultra-Large Sparse
// Models" (SameDay) §3.1; "Adapting GPU Software Stacks for Ultra-Large-Scale Sparse Attention
// Models: A Day-0 Engineering Guide" (GPUGuide) §3.1-§3.3.
#include "common.h"
#include "kernels.h"

namespace sa {

// Candidate sources of the selection.
//   kTokens:     candidate i is token position i; key row = slot of i.
//   kBlocks:     candidate j is block (page) j; key row = its physical page in the pooled
//                summary table (SameDay §3.1 coarse filtering over cached summaries).
//   kCandidates: candidate i is token (blocks[i / P] * P + i % P) of a kept block (fine stage).
enum { kTokens = 0, kBlocks = 1, kCandidates = 2 };

// Indexer key formats: bf16, E4M3 with one fp32 scale per row, MXFP8 (E4M3 with one E8M0
// exponent per 32 entries).
enum { kKeyBf16 = 0, kKeyE4M3 = 1, kKeyMx = 2 };

struct SeqCtx {
    int seq;
    int ctx;
    int ncand;
    const int32_t *pt;
    const int32_t *blocks;
};

__device__ __forceinline__ int ncand_of(int mode, int ctx, int lp, int block_k) {
    if (mode == kTokens) return ctx;
    const int nblk = (ctx + (1 << lp) - 1) >> lp;
    if (mode == kBlocks) return nblk;
    return min(block_k, nblk) << lp;
}

// Map candidate i to (logical position, key row); row < 0 when the candidate is not visible.
template <int MODE>
__device__ __forceinline__ void cand_row(const SeqCtx &s, int i, int lp, int &pos, int64_t &row) {
    const int P = 1 << lp;
    if (MODE == kTokens) {
        pos = i;
        row = (int64_t)s.pt[i >> lp] * P + (i & (P - 1));
    } else if (MODE == kBlocks) {
        pos = i;
        row = s.pt[i];
    } else {
        const int blk = s.blocks[i >> lp];
        pos = blk * P + (i & (P - 1));
        row = (blk >= 0 && pos < s.ctx) ? (int64_t)s.pt[blk] * P + (i & (P - 1)) : -1;
        if (blk < 0) pos = -1;
    }
}

// Indexer query fragments for one query row: A operands of the 16x16x32 MFMA for HT head
// tiles of 16 heads and KS k-steps of 32 entries. For E4M3 keys the d ordering inside each
// pair of k-steps is permuted so that a lane's 16 key bytes are contiguous; the query
// fragment follows the same order (the dot product does not depend on it).
template <int DIM, int HT, bool FP8>
struct IdxQuery {
    static constexpr int KS = DIM / 32;
    u32x4 a[HT][KS];
    float w[HT][4];

    __device__ __forceinline__ static int d_of(int s, int g) {
        // first entry of the 8 consecutive d's this lane group holds at k-step s
        return FP8 ? (64 * (s >> 1) + 16 * g + 8 * (s & 1)) : (32 * s + 8 * g);
    }

    __device__ __forceinline__ void load(const uint16_t *q_row, const float *w_row, int heads) {
        const int l = lane_id(), g = l >> 4;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + (l & 15);
            const int hc = min(h, heads - 1);  // loads stay unconditional; padding heads are zeroed
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 v = ldg16(q_row + (size_t)hc * DIM + d_of(s, g));
                a[ht][s] = h < heads ? v : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hh = 16 * ht + 4 * g + i;
                const float x = w_row[min(hh, heads - 1)];
                w[ht][i] = hh < heads ? x : 0.f;
            }
        }
    }
};

// Raw key fragment of one 16-candidate tile for one lane: the lane's token is l % 16, and it
// holds KS k-steps of 8 bf16 (or, for E4M3, KS/2 chunks of 16 codes).
template <int DIM, bool FP8>
struct KeyFrag {
    u32x4 v[FP8 ? DIM / 64 : DIM / 32];
    float scale;  // E4M3 row scale (loaded with the codes so that no later load waits on it)
    uint32_t mx;  // MXFP8: E8M0 exponent of the lane's block (see key_mx_scale)
};

template <int DIM, bool FP8, bool ROWSCALE = FP8>
__device__ __forceinline__ void load_key_frag(KeyFrag<DIM, FP8> &f, const uint8_t *keys,
                                              const float *key_scale, int64_t row) {
    const int g = lane_id() >> 4;
    constexpr int RB = FP8 ? DIM : DIM * 2;  // bytes per key row
    const uint8_t *p = keys + row * RB;
    if (FP8) {
#pragma unroll
        for (int c = 0; c < DIM / 64; ++c) f.v[c] = ldg16_stream(p + 64 * c + 16 * g);
        if (ROWSCALE) f.scale = key_scale[row];
    } else {
#pragma unroll
        for (int s = 0; s < DIM / 32; ++s) f.v[s] = ldg16_stream(p + 64 * s + 16 * g);
    }
}

// Coalesced key tile of 16 consecutive candidates, as the decode selection streams it: load x
// of lane l is the 16-byte chunk (l % CPR) of tile row (TPL * x + l / CPR), so every load of a
// wave covers whole rows (64 contiguous bytes per 4 lanes at least) instead of one 16-byte
// piece of 16 different rows. Streams of such loads with the nontemporal hint reach a higher
// HBM rate; a per-wave LDS transpose (tile_to_frag) then yields the MFMA fragments.
template <int DIM, bool FP8>
struct KeyTile {
    static constexpr int RB = FP8 ? DIM : 2 * DIM;  // bytes per key row
    static constexpr int CPR = RB / 16;             // 16-byte chunks per row
    static constexpr int NL = RB / 64;              // loads per lane per tile
    static constexpr int TPL = 64 / CPR;            // tile rows covered by one load
    static constexpr int RPB = 16 / CPR;            // tile rows per 256-byte LDS line
    u32x4 v[NL];
    float scale;  // E4M3 scale of the lane's own candidate (lane l % 16)
    uint32_t mx;  // MXFP8: E8M0 exponent of block l / 16 of the lane's own candidate

    // LDS slot (16-byte units) of chunk c of tile row r. The XOR swizzle makes both access
    // patterns bank-conflict free: the row-major writes, and the fragment reads in which 16
    // lanes read the same chunk of 16 different rows.
    __device__ static __forceinline__ int slot(int r, int c) {
        return (r / RPB) * 16 + (r % RPB) * CPR + (c ^ ((r / RPB) % CPR));
    }
};

// Tile (row-major chunks) -> fragment (lane l: candidate l % 16, chunks 4x + l / 16) through the
// wave's own 16-row LDS staging area. Only this wave touches `stage`, and LDS operations of a
// wave complete in order, so no barrier is needed.
template <int DIM, bool FP8>
__device__ __forceinline__ void tile_to_frag(const KeyTile<DIM, FP8> &t, u32x4 *stage,
                                             KeyFrag<DIM, FP8> &f) {
    using T = KeyTile<DIM, FP8>;
    const int l = lane_id();
#pragma unroll
    for (int x = 0; x < T::NL; ++x) stage[T::slot(T::TPL * x + l / T::CPR, l % T::CPR)] = t.v[x];
#pragma unroll
    for (int x = 0; x < T::NL; ++x) f.v[x] = stage[T::slot(l & 15, 4 * x + (l >> 4))];
    f.scale = t.scale;
    f.mx = t.mx;
}

// Score of the lane's candidate (lane l % 16; every lane of the 4 groups gets the same value).
template <int DIM, int HT, bool FP8>
__device__ __forceinline__ float score_tile(const IdxQuery<DIM, HT, FP8> &q,
                                            const KeyFrag<DIM, FP8> &f) {
    constexpr int KS = DIM / 32;
    f32x4 acc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 b;
        if (FP8) {
            const u32x4 raw = f.v[s >> 1];
            const int base = (s & 1) * 2;
            const u32x2 lo = e4m3x4_to_bf16(raw[base]);
            const u32x2 hi = e4m3x4_to_bf16(raw[base + 1]);
            b = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            b = f.v[s];
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(q.a[ht][s], b, acc[ht]);
    }
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(q.w[ht][i], relu(acc[ht][i]), part);
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    return part;
}

// ------------------------------------------------------------------ MXFP8 indexer
// [CANN] §3: the indexer runs in MXFP8, with per-group dynamic quantization (groups of 32) of
// the query and keys stored with one E8M0 exponent per 32 entries. On gfx950 one block-scaled
// MFMA (16x16x128, E4M3 x E4M3, E8M0 scales per 32-entry block) takes a 16-head x 16-token
// tile over the whole 128-entry head dimension: no conversion of key codes and no per-token
// scale multiply. The query is quantized once per workgroup, in registers.
//
// Lane l of head tile ht holds head h = 16 ht + l%16 and the entries 16 g .. 16 g + 15 (lo) and
// 64 + 16 g .. 64 + 16 g + 15 (hi) of its row, g = l / 16: these lie in blocks g/2 and 2 + g/2,
// so the block maxima come from the lane and its partner l ^ 16. The MFMA wants, in lane l, the
// exponent of block g, which lanes of group 2 (block 1) or 0 (block 2) computed. d_I = 64 keeps
// hi zero and blocks 2, 3 at scale 1.
template <int DIM, int HT>
struct MxQuery {
    u32x4 lo[HT], hi[HT];
    uint32_t sc[HT];
    float w[HT][4];

    // 16 bf16 (two 16-byte words) -> 16 E4M3 codes of v / 2^x
    __device__ static __forceinline__ u32x4 encode16(u32x4 a, u32x4 b, int x) {
        u32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w0 = j < 2 ? a[2 * j] : b[2 * j - 4];
            const uint32_t w1 = j < 2 ? a[2 * j + 1] : b[2 * j - 3];
            r[j] = e4m3_rne(ldexpf(bf16_lo(w0), -x)) | (e4m3_rne(ldexpf(bf16_hi(w0), -x)) << 8) |
                   (e4m3_rne(ldexpf(bf16_lo(w1), -x)) << 16) |
                   (e4m3_rne(ldexpf(bf16_hi(w1), -x)) << 24);
        }
        return r;
    }
    // largest magnitude of 16 bf16, as a bit pattern with the sign cleared (monotone in value)
    __device__ static __forceinline__ uint32_t amax16(u32x4 a, u32x4 b) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = max(m, max(a[j] & 0x7FFFu, (a[j] >> 16) & 0x7FFFu));
            m = max(m, max(b[j] & 0x7FFFu, (b[j] >> 16) & 0x7FFFu));
        }
        return m;
    }

    __device__ __forceinline__ void load(const uint16_t *q_row, const float *w_row, int heads) {
        const int l = lane_id(), g = l >> 4;
        const u32x4 z = {0u, 0u, 0u, 0u};
        // all loads first (unconditional, padding heads read a valid row and are zeroed), so
        // that one wait covers them
        u32x4 raw[HT][4];
        float wr[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + (l & 15);
            const uint16_t *p = q_row + (size_t)min(h, heads - 1) * DIM + 16 * g;
#pragma unroll
            for (int c = 0; c < (DIM == 128 ? 4 : 2); ++c) raw[ht][c] = ldg16(p + (c >> 1) * 64 + (c & 1) * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) wr[ht][i] = w_row[min(16 * ht + 4 * g + i, heads - 1)];
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + (l & 15);
            const bool ok = h < heads;
            const u32x4 a0 = ok ? raw[ht][0] : z, a1 = ok ? raw[ht][1] : z;
            const u32x4 b0 = (DIM == 128 && ok) ? raw[ht][2] : z;
            const u32x4 b1 = (DIM == 128 && ok) ? raw[ht][3] : z;
            uint32_t m0 = amax16(a0, a1), m1 = amax16(b0, b1);
            m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 16, 64));
            m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16, 64));
            const int x0 = mx_block_exp(m0);  // block g / 2
            const int x1 = mx_block_exp(m1);  // block 2 + g / 2
            lo[ht] = encode16(a0, a1, x0);
            hi[ht] = DIM == 128 ? encode16(b0, b1, x1) : z;
            const int from2 = __shfl(x0, (l & 15) + 32, 64);  // block 1
            const int from0 = __shfl(x1, l & 15, 64);         // block 2
            int x;
            if (DIM == 128) x = g == 0 ? x0 : g == 1 ? from2 : g == 2 ? from0 : x1;
            else x = g == 0 ? x0 : g == 1 ? from2 : 0;
            sc[ht] = (uint32_t)(x + 127);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[ht][i] = 16 * ht + 4 * g + i < heads ? wr[ht][i] : 0.f;
        }
    }
};

// E8M0 exponent that lane l supplies for its token's key row: block l / 16. For d_I = 64 the
// blocks 2, 3 hold zero codes, and lanes 32..63 repeat the exponents of blocks 0, 1 (any finite
// scale of a zero block adds nothing). No select follows the load, so nothing that consumes it
// is forced to wait where it would be placed.
template <int DIM>
__device__ __forceinline__ uint32_t key_mx_scale(const uint8_t *key_mx, int64_t row) {
    const int g = lane_id() >> 4;
    return key_mx[row * (DIM / 32) + (g % (DIM / 32))];
}

// MXFP8 score of the lane's candidate (lane l % 16; every lane of the 4 groups gets the same
// value). The fragment holds the token's codes in the E4M3 layout of KeyFrag (chunk g, and for
// d_I = 128 chunk 4 + g) and its block exponent in mx.
template <int DIM, int HT>
__device__ __forceinline__ float score_tile_mx(const MxQuery<DIM, HT> &q, const u32x4 *kv,
                                               uint32_t mx) {
    const u32x4 khi = DIM == 128 ? kv[1] : u32x4{0u, 0u, 0u, 0u};
    float part = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const f32x4 acc = mfma_mx16x16x128(q.lo[ht], q.hi[ht], q.sc[ht], kv[0], khi, mx,
                                           f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(q.w[ht][i], relu(acc[i]), part);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    return part;
}

// ============================================================== scores to HBM (sa_index_score)
// Grid: (row, chunk of 1024 candidates). 4 waves; each wave walks 16-token tiles.
constexpr int kScoreChunk = 1024;

template <int DIM, int HT, int KF>
__global__ __launch_bounds__(256) void k_index_score(ScoreArgs a) {
    constexpr bool FP8 = KF != kKeyBf16, MX = KF == kKeyMx;
    const int row = blockIdx.y;
    int seq, qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int ctx = a.ctx_lens[seq];
    const int nvis = ctx - qlen + qoff + 1;  // positions 0 .. row position
    const int64_t c0 = (int64_t)blockIdx.x * kScoreChunk;
    float *out = a.scores + (int64_t)row * a.ld;
    for (int64_t t = c0 + threadIdx.x; t < min(c0 + kScoreChunk, a.ld); t += 256)
        if (t >= nvis) out[t] = -__builtin_inff();
    const int c1 = (int)min(c0 + kScoreChunk, (int64_t)nvis);
    if (c1 <= c0) return;

    IdxQuery<DIM, HT, FP8> q;
    MxQuery<DIM, HT> qm;
    if constexpr (MX) qm.load(a.q_idx + (size_t)row * a.heads * DIM, a.w + (size_t)row * a.heads, a.heads);
    else q.load(a.q_idx + (size_t)row * a.heads * DIM, a.w + (size_t)row * a.heads, a.heads);
    SeqCtx s{seq, ctx, ctx, a.page_table + (int64_t)seq * a.pages_per_seq, nullptr};
    const int l = lane_id();
    const int ntiles = (c1 - (int)c0 + 15) >> 4;
    for (int tt = wave_id(); tt < ntiles; tt += 4) {
        int i = (int)c0 + 16 * tt + (l & 15);
        const bool valid = i < c1;
        if (!valid) i = (int)c0;
        int pos;
        int64_t krow;
        cand_row<kTokens>(s, i, a.lp, pos, krow);
        KeyFrag<DIM, FP8> f;
        float sc;
        if constexpr (MX) {
            load_key_frag<DIM, true, false>(f, a.keys, nullptr, krow);
            sc = score_tile_mx<DIM, HT>(qm, f.v, key_mx_scale<DIM>(a.key_mx, krow));
        } else {
            load_key_frag<DIM, FP8>(f, a.keys, a.key_scale, krow);
            sc = score_tile<DIM, HT, FP8>(q, f);
            if (FP8) sc *= f.scale;
        }
        if (valid && l < 16) out[i] = sc;
    }
}

// ============================================================= prefill scores (dense GEMM)
// Scores of many query rows of one sequence against all of its keys: a GEMM over
// (query row, head) x token with d_I as the contraction, followed by ReLU, the head weights and
// the sum over heads ([CANN] §2.1; [Domestic] §3.3: prefill selects over the whole range at
// once and is dominated by dense matrix work).
//
// Workgroup: 8 query rows of one sequence (one per wave) x a range of kPfTokens tokens. A wave
// keeps its row's query fragments for all heads in registers (A operand of
// v_mfma_f32_32x32x16_bf16: 32 heads x 16 dims per fragment) and multiplies them with 64-token
// key tiles (B operand: 16 dims x 32 tokens) that the workgroup stages in LDS, double
// buffered: E4M3 keys are widened to bf16 on the way (exact). The epilogue applies ReLU and
// the weights to the 32x32 (head x token) accumulators, sums over heads in registers and with
// the partner lane, and stores 64 consecutive scores per tile. Positions past a row's own
// position get -inf.
constexpr int kPfRows = 8;
constexpr int kPfTile = 128;
constexpr int kPfTokens = 8192;

template <int DIM, int MT, bool FP8>
__global__ __launch_bounds__(512, 1) void k_prefill_score(ScoreArgs a) {
    constexpr int RB = 2 * DIM;                 // LDS bytes per staged key row (bf16)
    constexpr int CPR = RB / 16;                // 16-byte chunks per staged row
    constexpr int RPB = 16 / CPR;               // staged rows per 256-byte LDS line
    constexpr int KS = DIM / 16;                // k-steps
    constexpr int GRB = FP8 ? DIM : 2 * DIM;    // global bytes per key row
    constexpr int GCH = kPfTile * GRB / 16;     // global 16-byte chunks per tile
    constexpr int GPT = (GCH + 511) / 512;      // chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t kt[2][kPfTile * RB];
    __shared__ float s_scale[2][kPfTile];
    __shared__ int32_t s_page[kPfTokens + 1];  // physical page of each page the range touches
    __shared__ int s_loc[4];
    auto slot = [](int r, int c) { return (r / RPB) * 16 + (r % RPB) * CPR + (c ^ ((r / RPB) % CPR)); };

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    // ---- (sequence, row block) of this workgroup: row blocks counted per sequence
    if (tid < 64) {
        uint32_t base = 0;
        int fs = -1, fb = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int b = b0 + l;
            uint32_t nb = 0;
            if (b < a.num_seqs) nb = (uint32_t)(a.q_indptr[b + 1] - a.q_indptr[b] + kPfRows - 1) / kPfRows;
            const uint32_t incl = wave_incl_scan(nb);
            const uint32_t excl = base + incl - nb;
            if (b < a.num_seqs && blockIdx.x >= excl && blockIdx.x < excl + nb) {
                fs = b;
                fb = blockIdx.x - excl;
            }
            base += __shfl(incl, 63, 64);
        }
        const uint64_t m = __ballot(fs >= 0);
        const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
        fs = __shfl(fs, src, 64);
        fb = __shfl(fb, src, 64);
        if (tid == 0) {
            s_loc[0] = m ? fs : -1;
            s_loc[1] = fb;
        }
    }
    __syncthreads();
    if (s_loc[0] < 0) return;
    const int seq = s_loc[0];
    const int q0 = a.q_indptr[seq], q1 = a.q_indptr[seq + 1];
    const int ctx = a.ctx_lens[seq];
    const int row0 = q0 + kPfRows * s_loc[1];
    const int row = row0 + w;
    const bool live = row < q1;
    const int pos0 = ctx - (q1 - q0);                   // position of the sequence's first row
    const int p_row = live ? pos0 + (row - q0) : -1;    // last visible position of this row
    const int p_max = pos0 + (min(q1, row0 + kPfRows) - 1 - q0);
    const int64_t tb0 = (int64_t)blockIdx.y * kPfTokens;
    const int64_t tb1 = min(a.ld, tb0 + kPfTokens);
    const int32_t *pt = a.page_table + (int64_t)seq * a.pages_per_seq;
    const int P = 1 << a.lp;
    float *out = live ? a.scores + (int64_t)row * a.ld : nullptr;

    // ---- query fragments and head weights of this wave's row
    u32x4 qa[MT][KS];
    float wv[MT][4][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int hd = 32 * mt + (l & 31);
        const uint16_t *qr = a.q_idx + ((int64_t)(live ? row : q0) * a.heads + hd) * DIM + 8 * (l >> 5);
#pragma unroll
        for (int s = 0; s < KS; ++s) qa[mt][s] = (live && hd < a.heads) ? ldg16(qr + 16 * s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hh = 32 * mt + 8 * j + 4 * (l >> 5) + i;
                wv[mt][j][i] = (live && hh < a.heads) ? a.w[(int64_t)row * a.heads + hh] : 0.f;
            }
    }

    // ---- tiles with work: [tb0, t_end) where t_end covers the last visible position of the
    //      workgroup's rows; later columns only get -inf
    const int64_t t_end = min(tb1, (int64_t)p_max + 1);
    const int ntiles = t_end > tb0 ? (int)((t_end - tb0 + kPfTile - 1) / kPfTile) : 0;
    // pages of the tokens [tb0, ctx) that the tiles can touch, so that no key address waits
    // on a global load
    const int pfirst = (int)(tb0 >> a.lp);
    if (ntiles > 0) {
        const int plast = (int)((min(tb1, (int64_t)ctx) - 1) >> a.lp);
        for (int j = tid; j <= plast - pfirst; j += 512) s_page[j] = pt[pfirst + j];
    }
    // query fragments, weights and the page table complete before the loop, so that inside it
    // the only vector-memory loads in flight are key tiles
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // key tiles move global -> registers one tile ahead -> LDS (double buffered)
    u32x4 stA[GPT];
    float scA = 1.f;
    auto krow_of = [&](int64_t tok) -> int64_t {  // past the sequence: its last resident row
        if (tok >= ctx) tok = ctx - 1;
        return (int64_t)s_page[(int)(tok >> a.lp) - pfirst] * P + (tok & (P - 1));
    };
    // t beyond the last tile reloads the last tile (harmless), so the loads are unconditional
    auto load = [&](int t, u32x4 (&stg)[GPT], float &scl) {
        const int64_t t0 = tb0 + (int64_t)min(t, ntiles - 1) * kPfTile;
#pragma unroll
        for (int g = 0; g < GPT; ++g) {
            const int c = min(tid + 512 * g, GCH - 1);
            stg[g] = ldg16(a.keys + krow_of(t0 + c / (GRB / 16)) * GRB + 16 * (c % (GRB / 16)));
        }
        if (FP8) scl = a.key_scale[krow_of(t0 + (tid & (kPfTile - 1)))];
    };
    auto store = [&](int buf, const u32x4 (&stg)[GPT], float scl) {
#pragma unroll
        for (int g = 0; g < GPT; ++g) {
            const int c = tid + 512 * g;
            if (c >= GCH) continue;
            const int r = c / (GRB / 16), gc = c % (GRB / 16);
            u32x4 *dst = reinterpret_cast<u32x4 *>(kt[buf]);
            if (FP8) {  // 16 codes -> 16 bf16 = staged chunks 2 gc, 2 gc + 1
                const u32x2 lo0 = e4m3x4_to_bf16(stg[g][0]), hi0 = e4m3x4_to_bf16(stg[g][1]);
                const u32x2 lo1 = e4m3x4_to_bf16(stg[g][2]), hi1 = e4m3x4_to_bf16(stg[g][3]);
                dst[slot(r, 2 * gc)] = u32x4{lo0[0], lo0[1], hi0[0], hi0[1]};
                dst[slot(r, 2 * gc + 1)] = u32x4{lo1[0], lo1[1], hi1[0], hi1[1]};
            } else {
                dst[slot(r, gc)] = stg[g];
            }
        }
        if (FP8 && tid < kPfTile) s_scale[buf][tid] = scl;
    };
    auto compute = [&](int t) {
        constexpr int NN = kPfTile / 32;  // 32-token MFMA tiles per key tile
        const int buf = t & 1;
        const int64_t t0 = tb0 + (int64_t)t * kPfTile;
        if (!live) return;
        float v[NN];
        if (t0 <= p_row) {
            const u32x4 *kb = reinterpret_cast<const u32x4 *>(kt[buf]);
#pragma unroll
            for (int nt = 0; nt < NN; ++nt) {
                f32x16 acc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const u32x4 b = kb[slot(32 * nt + (l & 31), 2 * s + (l >> 5))];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16(qa[mt][s], b, acc[mt]);
                }
                float x = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x = fmaf(wv[mt][j][i], relu(acc[mt][4 * j + i]), x);
                x = sum_xor32(x);
                if (FP8) x *= s_scale[buf][32 * nt + (l & 31)];
                v[nt] = x;
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < NN; ++nt) v[nt] = 0.f;
        }
        // 64 consecutive tokens per store: lanes 0..31 hold MFMA tile 2p, lanes 32..63 tile 2p+1
#pragma unroll
        for (int pp = 0; pp < NN / 2; ++pp) {
            const int64_t tok = t0 + 64 * pp + l;
            const float x = l < 32 ? v[2 * pp] : v[2 * pp + 1];
            // streamed out (nontemporal): the row Top-K reads them once, and they do not
            // displace reused lines from the caches
            if (tok < tb1) __builtin_nontemporal_store(tok <= p_row ? x : -__builtin_inff(), &out[tok]);
        }
    };
    // step t: tile t + 1 moves global -> registers while tile t is computed, then registers
    // -> the other LDS buffer. Loads are unconditional (a step past the last tile reloads the
    // last tile), so the wait before the LDS store covers exactly these loads.
    if (ntiles > 0) {
        load(0, stA, scA);
        store(0, stA, scA);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        load(t + 1, stA, scA);
        compute(t);
        if (t + 1 < ntiles) store((t + 1) & 1, stA, scA);
        __syncthreads();
    }
    // ---- columns past every row of the workgroup
    if (live)
        for (int64_t tok = tb0 + (int64_t)ntiles * kPfTile + l; tok < tb1; tok += 64)
            __builtin_nontemporal_store(-__builtin_inff(), &out[tok]);
}

// ================================================================ decode selection (fused)
// One workgroup per chunk of a sequence's candidates; all chunks of all sequences are
// co-resident (the grid is sized within the device's resident capacity). Scores never leave
// LDS: they become order-preserving keys and an exact radix select runs over the sequence
// with per-pass global histograms and a barrier per pass. Selected candidates are written in
// ascending position order; ties at the threshold go to the lower positions.
constexpr int kSelThreads = 512;
static_assert(kListCap % kSelThreads == 0, "whole list entries per thread");
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 2048;

struct alignas(16) SelShared {
    uint32_t hist[kHistBins];
    uint32_t scan[2 * kSelWaves + 1];
    uint32_t res[8];
    uint32_t grp[2];
};

// Per-chunk address table in LDS (built once, so the key stream never waits on a page-table
// load): for kTokens / kCandidates one entry per page touched by the chunk (row of the page's
// first token, and for kCandidates the kept block id); for kBlocks one row per candidate.
template <int MODE>
struct ChunkRows {
    int first;          // first page (kTokens / kCandidates) touched by the chunk
    int32_t *row;       // LDS
    int32_t *blk;       // LDS (kCandidates)

    __device__ __forceinline__ void cand(const SeqCtx &s, int i, int c0, int lp, int &pos,
                                         int64_t &r) const {
        const int P = 1 << lp;
        if (MODE == kTokens) {
            pos = i;
            r = (int64_t)row[(i >> lp) - first] + (i & (P - 1));
        } else if (MODE == kBlocks) {
            pos = i;
            r = row[i - c0];
        } else {
            const int j = (i >> lp) - first;
            const int b = blk[j];
            pos = b >= 0 ? b * P + (i & (P - 1)) : -1;
            r = (b >= 0 && pos < s.ctx) ? (int64_t)row[j] + (i & (P - 1)) : -1;
        }
    }
};

// Row of the first candidate of a 16-aligned tile when all 16 rows are contiguous (pages of at
// least 16 tokens, modes kTokens / kCandidates); a tile of a dropped block reads rows 0..15.
template <int MODE>
__device__ __forceinline__ int64_t tile_base_row(const ChunkRows<MODE> &cr, int i0, int lp) {
    const int P = 1 << lp;
    const int j = (i0 >> lp) - cr.first;
    if (MODE == kCandidates && cr.blk[j] < 0) return 0;
    return (int64_t)cr.row[j] + (i0 & (P - 1));
}

__host__ __device__ inline int chunk_table_entries(int mode, int chunk, int lp) {
    return mode == kBlocks ? chunk : (chunk >> lp) + 2;
}

// ---- locate a workgroup's (sequence, chunk): chunk counts prefix over sequences, groups_of(ctx)
//      giving a sequence's workgroups. Returns false for grid padding (never co-waited on).
template <class GF>
__device__ __forceinline__ bool select_locate(const SelectArgs &a, GF groups_of, SelShared &sh,
                                              int &seq, int &chunk, int &G, int &ctx) {
    const int tid = threadIdx.x, l = lane_id();
    if (tid < 64) {
        uint32_t base = 0;
        int found_seq = -1, found_chunk = 0, found_G = 0, found_ctx = 0;
        for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
            const int b = b0 + l;
            uint32_t nchunks = 0;
            int ctx_b = 0;
            if (b < a.num_seqs) {
                ctx_b = a.ctx_lens[b];
                // a sequence that reuses another's selection has no workgroups
                nchunks = (a.reuse && a.reuse[b] >= 0) ? 0u : (uint32_t)groups_of(ctx_b);
            }
            const uint32_t incl = wave_incl_scan(nchunks);
            const uint32_t excl = base + incl - nchunks;
            if (b < a.num_seqs && blockIdx.x >= excl && blockIdx.x < excl + nchunks) {
                found_seq = b;
                found_chunk = blockIdx.x - excl;
                found_G = nchunks;
                found_ctx = ctx_b;
            }
            base += __shfl(incl, 63, 64);
        }
        // exactly one lane (over all iterations) found it
        const uint64_t m = __ballot(found_seq >= 0);
        const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
        const int fs = __shfl(found_seq, src, 64);
        const int fc = __shfl(found_chunk, src, 64);
        const int fg = __shfl(found_G, src, 64);
        const int fx = __shfl(found_ctx, src, 64);
        if (tid == 0) {
            sh.res[0] = m ? fs : 0xFFFFFFFFu;
            sh.res[1] = fc;
            sh.res[2] = fg;
            sh.res[3] = fx;  // the sequence's length, already loaded here
        }
    }
    __syncthreads();
    if (sh.res[0] == 0xFFFFFFFFu) return false;
    seq = sh.res[0];
    chunk = sh.res[1];
    G = sh.res[2];
    ctx = (int)sh.res[3];
    __syncthreads();  // sh.res is reused after this
    return true;
}

// Everything a workgroup does once it knows its (sequence, chunk): the chunk's address table,
// its scores as keys in LDS, the radix select across the G workgroups of the sequence (record
// ss, barriers numbered from nbar on), the ordered emission and the leave step. ok0 = false
// carries an expired wait of an earlier phase into this one's failure flag.
template <int DIM, int HT, int KF, int MODE>
__device__ __forceinline__ void select_run(const SelectArgs &a, int seq, int chunk, int G, int ctx,
                                          SelSync *ss, uint32_t &nbar, bool ok0, uint32_t *s_key,
                                          SelShared &sh, u32x4 (*s_stage)[256]) {
    constexpr bool FP8 = KF != kKeyBf16, MX = KF == kKeyMx;
    const int tid = threadIdx.x, l = lane_id();
    const int clen = a.chunk;
    SeqCtx s;
    s.seq = seq;
    s.ctx = ctx;
    s.ncand = ncand_of(MODE, s.ctx, a.lp, a.block_k);
    s.pt = a.page_table + (int64_t)seq * a.pages_per_seq;
    s.blocks = MODE == kCandidates ? a.blocks + (int64_t)seq * a.block_k : nullptr;
    const int c0 = chunk * clen;
    const int c1 = min(c0 + clen, s.ncand);
    const int cnt = max(0, c1 - c0);

    // ---- address table of the chunk
    ChunkRows<MODE> cr;
    cr.first = c0 >> a.lp;
    cr.row = reinterpret_cast<int32_t *>(s_key + a.chunk);
    cr.blk = cr.row + chunk_table_entries(MODE, a.chunk, a.lp);
    if (cnt > 0) {
        const int P = 1 << a.lp;
        if (MODE == kBlocks) {
            for (int i = tid; i < cnt; i += kSelThreads) cr.row[i] = s.pt[c0 + i];
        } else {
            const int npg = ((c1 - 1) >> a.lp) - cr.first + 1;
            for (int j = tid; j < npg; j += kSelThreads) {
                const int pg = cr.first + j;
                if (MODE == kTokens) {
                    cr.row[j] = s.pt[pg] * P;
                } else {
                    // agent scope: in the fused two-stage launch the list was written by
                    // workgroups on other XCDs moments ago
                    const int b = (int)ld_agent(reinterpret_cast<const uint32_t *>(s.blocks + pg));
                    cr.blk[j] = b;
                    cr.row[j] = b >= 0 ? s.pt[b] * P : -1;
                }
            }
        }
    }
    // the first radix pass's histogram (top 11 key bits) is built while the keys stream in
    for (int i = tid; i < kHistBins; i += kSelThreads) sh.hist[i] = 0u;
    __syncthreads();

    // ---- scores of this chunk -> LDS keys (0 = not a candidate)
    if (cnt > 0) {
        IdxQuery<DIM, HT, FP8> q;
        MxQuery<DIM, HT> qm;
        if constexpr (MX) qm.load(a.q_idx + (size_t)seq * a.heads * DIM, a.w + (size_t)seq * a.heads, a.heads);
        else q.load(a.q_idx + (size_t)seq * a.heads * DIM, a.w + (size_t)seq * a.heads, a.heads);
        const int ntiles = (cnt + 15) >> 4;
        const int w = wave_id();
        const int my_tiles = ntiles > w ? (ntiles - w + kSelWaves - 1) / kSelWaves : 0;
        using KT = KeyTile<DIM, FP8>;
        // tiles in flight per wave: 4 KiB of keys, 8 KiB for MXFP8 (whose tiles cost the least
        // compute). With every CU pulling keys at once, more requests in flight only lengthen
        // the memory queues: back to back at decode32k, 4 KiB take 55.7 us per launch against
        // 56.5 with 8 KiB, and 16 or 24 KiB were slower still.
        constexpr int kPre = (MX ? 8 : 4) / KT::NL;
        KT f[kPre];
        u32x4 *stage = s_stage[w];
        const bool contiguous = MODE != kBlocks && a.lp >= 4;
        auto lrow = [&](int i) -> int64_t {  // load row of candidate i (row 0 if invalid)
            if (i >= c1) i = c0;
            int pos;
            int64_t r;
            cr.cand(s, i, c0, a.lp, pos, r);
            return r < 0 ? 0 : r;
        };
        // Every step issues the same loads: a step past the wave's last tile reads row 0 of the
        // key table (the same bytes for every such step of the launch, so L2 serves them),
        // and loads whose value is not needed read a valid row and are discarded by the
        // consumer. The number of loads issued after a tile's own is then the same on every
        // path, so the wait before each tile is exact and kPre tiles stay in flight; a load
        // behind a branch would make the compiler wait for every outstanding load instead.
        auto issue = [&](int slot, int k) {
            // all-ones for a real tile, zero past the last one; opaque to the compiler, which
            // would otherwise turn the masking into branches around the loads
            int64_t keep = -(int64_t)(k < my_tiles);
            asm volatile("" : "+v"(keep));
            k = min(k, my_tiles - 1);
            const int i0 = c0 + 16 * (w + k * kSelWaves);
            const int64_t base = contiguous ? tile_base_row(cr, i0, a.lp) : 0;
#pragma unroll
            for (int x = 0; x < KT::NL; ++x) {
                const int tr = KT::TPL * x + l / KT::CPR;
                const int64_t row = (contiguous ? base + tr : lrow(i0 + tr)) & keep;
                f[slot].v[x] = ldg16_stream(a.keys + row * KT::RB + 16 * (l % KT::CPR));
            }
            if (FP8) {
                const int i = i0 + (l & 15);
                int pos;
                int64_t r;
                cr.cand(s, i < c1 ? i : c0, c0, a.lp, pos, r);
                // a candidate without a row (a dropped block) reads row 0; its key is discarded
                const int64_t rr = (r >= 0 ? r : 0) & keep;
                if (MX) f[slot].mx = key_mx_scale<DIM>(a.key_mx, rr);
                else f[slot].scale = a.key_scale[rr];
            }
        };
        if (my_tiles > 0) {
#pragma unroll
            for (int k = 0; k < kPre; ++k) issue(k, k);
            for (int k0 = 0; k0 < my_tiles; k0 += kPre) {
#pragma unroll
                for (int j = 0; j < kPre; ++j) {
                    const int k = k0 + j;
                    KeyFrag<DIM, FP8> fr;
                    tile_to_frag<DIM, FP8>(f[j], stage, fr);
                    // take the tile's scale word here, before the next load into its slot: a
                    // plain copy would be placed after that load is issued, and the register
                    // rotation it causes waits for every outstanding load
                    if constexpr (MX) asm volatile("v_mov_b32 %0, %1" : "=v"(fr.mx) : "v"(f[j].mx));
                    else if constexpr (FP8) asm volatile("v_mov_b32 %0, %1" : "=v"(fr.scale) : "v"(f[j].scale));
                    issue(j, k + kPre);
                    if (k < my_tiles) {
                        const int tt = w + k * kSelWaves;
                        const int li = 16 * tt + (l & 15);
                        float sc;
                        if constexpr (MX) {
                            sc = score_tile_mx<DIM, HT>(qm, fr.v, fr.mx);
                        } else {
                            sc = score_tile<DIM, HT, FP8>(q, fr);
                            if (FP8) sc *= fr.scale;
                        }
                        if (l < 16 && c0 + li < c1) {
                            bool ok = true;
                            if (MODE == kCandidates) {
                                int pos;
                                int64_t r;
                                cr.cand(s, c0 + li, c0, a.lp, pos, r);
                                ok = r >= 0;
                            }
                            const uint32_t key = ok ? float_key(sc) : 0u;
                            s_key[li] = key;
                            if (key) atomicAdd(&sh.hist[key >> 21], 1u);
                        }
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- radix select over the sequence
    uint32_t *s_base = reinterpret_cast<uint32_t *>(s_stage);  // the transpose area is free now
    uint32_t prefix = 0;
    int pbits = 0;
    uint32_t need = 0, total = 0;
    bool exact = false;  // every candidate in the threshold bin is selected
    uint32_t listn = 0;  // > 0: the threshold bin of the first pass is resolved through the list
    bool ok = ok0;  // false: a wait of an earlier stage expired
    for (int pass = 0; pass < 3; ++pass) {
        const int bits = pass < 2 ? 11 : 10;
        const int shift = 32 - pbits - bits;
        const int nb = 1 << bits;
        if (pass > 0) {  // pass 0's histogram was built with the keys
            for (int i = tid; i < kHistBins; i += kSelThreads) sh.hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < cnt; i += kSelThreads) {
                const uint32_t k = s_key[i];
                if (k == 0u) continue;
                if ((k >> (32 - pbits)) != prefix) continue;
                atomicAdd(&sh.hist[(k >> shift) & (nb - 1)], 1u);
            }
            __syncthreads();
        }
        uint32_t *gh = ss->hist[pass];
        // pass 0 keeps what each bin held before this workgroup's addition: if the bin turns
        // out to be the threshold bin, that is where this workgroup's candidates in it go in
        // the sequence's list (no further allocation round trip)
        for (int i = tid; i < nb; i += kSelThreads) {
            const uint32_t c = sh.hist[i];
            if (pass == 0) s_base[i] = c ? fetch_add_agent(&gh[i], c) : 0u;
            else if (c) add_agent(&gh[i], c);
        }
        ok = group_barrier(&ss->count, G, a.err, nbar, a.spin_limit) && ok;
        // suffix scan of the global histogram: thread t owns bins [nb - 4(t+1), nb - 4t). In
        // pass 0 the same scan runs over this workgroup's own histogram, which gives its count
        // above the threshold bin.
        uint32_t hv[4], lv[4];
        uint32_t csum = 0, lsum = 0;
        const int top = nb - 4 * tid - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = top - j;
            hv[j] = b >= 0 ? ld_agent(&gh[b]) : 0u;
            lv[j] = (pass == 0 && b >= 0) ? sh.hist[b] : 0u;
            csum += hv[j];
            lsum += lv[j];
        }
        uint32_t tot, labove0;
        const uint32_t above0 = block_excl_scan2<kSelThreads>(csum, lsum, sh.scan, &tot, &labove0);
        if (pass == 0) {
            total = tot;
            need = min((uint32_t)a.k, tot);
        }
        if (need == 0u) break;
        if (tid == 0) {
            sh.res[3] = 0xFFFFFFFFu;
            sh.res[4] = 0u;
            sh.res[5] = 0u;
            sh.res[6] = 0u;
        }
        __syncthreads();
        uint32_t run = above0, lrun = labove0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (run < need && run + hv[j] >= need) {
                sh.res[3] = (uint32_t)(top - j);
                sh.res[4] = run;
                sh.res[5] = hv[j];
                sh.res[6] = lrun;  // pass 0: this workgroup's candidates above the bin
            }
            run += hv[j];
            lrun += lv[j];
        }
        __syncthreads();
        uint32_t T = sh.res[3];
        if (T >= (uint32_t)nb) {  // no threshold bin: only after an expired wait (partial counts)
            T = 0u;
            ok = false;
        }
        need -= sh.res[4];
        prefix = (prefix << bits) | T;
        pbits += bits;
        if (pass == 0 && sh.res[5] <= (uint32_t)kListCap) {
            listn = sh.res[5];  // resolved below with one more exchange
            break;
        }
        if (sh.res[5] == need) {
            exact = true;
            break;
        }
    }

    // ---- per-workgroup counts -> global offsets
    const int K = a.k;
    int32_t *out = a.idx_out + (int64_t)seq * K;
    int32_t *slots = a.slots_out ? a.slots_out + (int64_t)seq * K : nullptr;
    const uint32_t k_eff = min((uint32_t)K, total);
    if (k_eff > 0 && listn > 0) {
        // ---- the first pass's threshold bin holds few candidates. Each workgroup publishes
        //      how many of its candidates lie above the bin and appends its candidates in the
        //      bin to the sequence's list as composites (key << 32 | ~candidate). Composites are
        //      distinct, and a larger composite means a larger score or, for equal scores, a
        //      lower candidate index (= lower position). After one exchange every workgroup
        //      reads the list and finds the exact threshold composite in LDS.
        // this workgroup's candidates above the bin (found with the pass-0 scan)
        const uint32_t above_tot = sh.res[6];
        if (tid == 0) {
            st_agent(&ss->cnt[chunk][0], above_tot);
            sh.grp[0] = 0u;
        }
        __syncthreads();
        {
            // the list's order is irrelevant (every reader takes all of it), so each wave
            // appends the bin's candidates of AB rounds at consecutive slots: one ballot per
            // round, one LDS atomic per wave for all of them, and coalesced stores
            const uint32_t lbase = s_base[prefix];
            constexpr int AB = 8;  // rounds whose keys are read before any is used
            for (int r0 = 0; r0 < cnt; r0 += AB * kSelThreads) {
                uint32_t kk[AB];
#pragma unroll
                for (int u = 0; u < AB; ++u) kk[u] = s_key[min(r0 + u * kSelThreads + tid, cnt - 1)];
                uint64_t m[AB];
                uint32_t wtot = 0;
#pragma unroll
                for (int u = 0; u < AB; ++u) {
                    asm volatile("" : "+v"(kk[u]));  // keeps the reads above out of branches
                    const bool in_bin = r0 + u * kSelThreads + tid < cnt && kk[u] != 0u &&
                                        (kk[u] >> 21) == prefix;
                    m[u] = __ballot(in_bin);
                    wtot += (uint32_t)__popcll(m[u]);
                }
                if (wtot == 0) continue;
                uint32_t woff = 0;
                if (l == 0) woff = atomicAdd(&sh.grp[0], wtot);
                woff = __builtin_amdgcn_readfirstlane(woff);
#pragma unroll
                for (int u = 0; u < AB; ++u) {
                    if ((m[u] >> l) & 1ull) {
                        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[u], 0u));
                        const int i = r0 + u * kSelThreads + tid;
                        // below kListCap whenever every workgroup's counts are in (the bin holds
                        // at most kListCap); the test keeps a workgroup whose wait expired, and
                        // which saw only part of the histogram, inside the list
                        const uint32_t slot = lbase + woff + below;
                        if (slot < (uint32_t)kListCap)
                            st_agent64(&ss->list[slot],
                                       ((uint64_t)kk[u] << 32) | (uint32_t)~(uint32_t)(c0 + i));
                    }
                    woff += (uint32_t)__popcll(m[u]);
                }
            }
        }
        ok = group_barrier(&ss->count, G, a.err, nbar, a.spin_limit) && ok;
        // the list (at most kListCap entries) stays in registers: thread tid holds entries
        // tid + kSelThreads r; 0 marks an empty slot (list keys are never 0). All loads are
        // issued before the first is used.
        constexpr int LPT = kListCap / kSelThreads;
        uint64_t lc[LPT];
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const int j = tid + kSelThreads * r;
            lc[r] = j < (int)listn ? ld_agent64(&ss->list[j]) : 0ull;
        }
        const uint32_t Ah = tid < chunk ? ld_agent(&ss->cnt[tid][0]) : 0u;
        // the pass-0 histogram (the only one this path uses) was last read before the barrier
        // above: clear it for the next launch while the list loads are in flight
        for (int i = chunk * kSelThreads + tid; i < kHistBins; i += G * kSelThreads)
            st_agent(&ss->hist[0][i], 0u);
        uint32_t a_before;
        block_excl_scan<kSelThreads>(Ah, sh.scan, &a_before);
        // exact threshold among the list: radix passes over the composites' remaining bits
        uint64_t pre = prefix;
        int pb = 11;
        uint32_t lneed = need;
        for (;;) {
            const int bits = min(11, 64 - pb);
            const int shift = 64 - pb - bits;
            const int nb = 1 << bits;
            for (int i = tid; i < kHistBins; i += kSelThreads) sh.hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int r = 0; r < LPT; ++r) {
                const uint64_t c = lc[r];
                if (c != 0ull && (c >> (64 - pb)) == pre)
                    atomicAdd(&sh.hist[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
            }
            __syncthreads();
            uint32_t hv[4];
            uint32_t csum = 0;
            const int top = nb - 4 * tid - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int b = top - j;
                hv[j] = b >= 0 ? sh.hist[b] : 0u;
                csum += hv[j];
            }
            uint32_t tot;
            const uint32_t abv = block_excl_scan<kSelThreads>(csum, sh.scan, &tot);
            if (tid == 0) {
                sh.res[3] = 0xFFFFFFFFu;
                sh.res[4] = 0u;
                sh.res[5] = 0u;
            }
            __syncthreads();
            uint32_t run = abv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < lneed && run + hv[j] >= lneed) {
                    sh.res[3] = (uint32_t)(top - j);
                    sh.res[4] = run;
                    sh.res[5] = hv[j];
                }
                run += hv[j];
            }
            __syncthreads();
            lneed -= sh.res[4];
            // (no bin found: only on partial counts, see below)
            const uint32_t tb = sh.res[3] < (uint32_t)nb ? sh.res[3] : 0u;
            pre = (pre << bits) | tb;
            pb += bits;
            // with complete counts the bin holds exactly what is still needed once all 64 bits
            // are used (composites are distinct); the bound on pb also ends the loop for a
            // workgroup whose wait expired and which works on partial counts
            const bool whole = sh.res[5] == lneed || pb >= 64;
            __syncthreads();
            if (whole) break;
        }
        // the threshold composite: comparing the top pb bits with pre is the same test as
        // comparing the whole composite with thr. Every composite of the bin or above it is
        // at least 2^32 (keys of candidates are never 0), so a candidate is selected exactly
        // when its composite (key << 32 | ~index, key 0 for non-candidates) is at least thr.
        const uint64_t thr = pre << (64 - pb);
        // list candidates of earlier workgroups that are selected
        uint32_t tb = 0;
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const uint64_t c = lc[r];
            const uint32_t ci = ~(uint32_t)c;
            // candidates of earlier workgroups: below this chunk's first candidate c0 (an empty
            // slot, 0, is below thr)
            tb += c >= thr && ci < (uint32_t)c0;
        }
        uint32_t taken_before;
        block_excl_scan<kSelThreads>(tb, sh.scan, &taken_before);
        auto take = [&](uint32_t k, int i) -> bool {  // k = s_key[i]
            return (((uint64_t)k << 32) | (uint32_t)~(uint32_t)(c0 + i)) >= thr;
        };
        // ordered emission: thread t owns the local candidates [E t, E t + E). Each thread
        // counts its selected candidates (keys read eight at a time, unconditionally), one
        // block scan gives its first slot after the earlier workgroups' selections, and a
        // second walk writes them in position order.
        const int E = (cnt + kSelThreads - 1) / kSelThreads;
        const int e0 = min(cnt, tid * E), e1 = min(cnt, e0 + E);
        auto keys8 = [&](int b, uint32_t *kk) {
#pragma unroll
            for (int u = 0; u < 8; ++u) kk[u] = s_key[min(b + u, e1 - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                asm volatile("" : "+v"(kk[u]));  // keeps the reads above out of branches
                kk[u] = b + u < e1 ? kk[u] : 0u;
            }
        };
        uint32_t my_sel = 0;
        for (int b = e0; b < e1; b += 8) {
            uint32_t kk[8];
            keys8(b, kk);
#pragma unroll
            for (int u = 0; u < 8; ++u) my_sel += take(kk[u], b + u) ? 1u : 0u;
        }
        uint32_t tmp_tot;
        uint32_t dst = a_before + taken_before + block_excl_scan<kSelThreads>(my_sel, sh.scan, &tmp_tot);
        for (int b = e0; b < e1; b += 8) {
            uint32_t kk[8];
            keys8(b, kk);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (!take(kk[u], b + u)) continue;
                int pos;
                int64_t row;
                cr.cand(s, c0 + b + u, c0, a.lp, pos, row);
                if (dst < (uint32_t)K) {
                    st_agent(reinterpret_cast<uint32_t *>(out) + dst, (uint32_t)pos);
                    if (slots) st_agent(reinterpret_cast<uint32_t *>(slots) + dst, (uint32_t)row);
                }
                ++dst;
            }
        }
    } else if (k_eff > 0) {
        const int sh_bits = 32 - pbits;
        uint32_t above = 0, eq = 0;
        for (int i = tid; i < cnt; i += kSelThreads) {
            const uint32_t k = s_key[i];
            if (k == 0u) continue;
            const uint32_t p = k >> sh_bits;
            above += p > prefix;
            eq += p == prefix;
        }
        uint32_t tmp;
        above = wave_sum(above);
        eq = wave_sum(eq);
        __syncthreads();
        if (l == 0) {
            sh.scan[wave_id()] = above;
            sh.hist[wave_id()] = eq;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t A = 0, Eq = 0;
            for (int i = 0; i < kSelWaves; ++i) {
                A += sh.scan[i];
                Eq += sh.hist[i];
            }
            st_agent(&ss->cnt[chunk][0], A);
            st_agent(&ss->cnt[chunk][1], Eq);
        }
        ok = group_barrier(&ss->count, G, a.err, nbar, a.spin_limit) && ok;
        // prefix over the earlier workgroups of this sequence (chunk order = position order);
        // G <= kSelThreads, so thread h reads the record of workgroup h
        uint32_t Ah = 0, Eh = 0;
        if (tid < chunk) {
            Ah = ld_agent(&ss->cnt[tid][0]);
            Eh = ld_agent(&ss->cnt[tid][1]);
        }
        uint32_t eq_before;
        const uint32_t e_excl = block_excl_scan<kSelThreads>(Eh, sh.scan, &eq_before);
        const uint32_t taken = exact ? Eh : (need > e_excl ? min(Eh, need - e_excl) : 0u);
        uint32_t off;
        block_excl_scan<kSelThreads>(Ah + taken, sh.scan, &off);
        // ordered emission: thread t owns local candidates [t*E, t*E + E)
        const int E = (cnt + kSelThreads - 1) / kSelThreads;
        const int i0 = min(cnt, tid * E), i1 = min(cnt, i0 + E);
        uint32_t my_eq = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = s_key[i];
            my_eq += (k != 0u) && ((k >> sh_bits) == prefix);
        }
        const uint32_t eq_rank0 = eq_before + block_excl_scan<kSelThreads>(my_eq, sh.scan, &tmp);
        uint32_t my_sel = 0;
        {
            uint32_t er = eq_rank0;
            for (int i = i0; i < i1; ++i) {
                const uint32_t k = s_key[i];
                if (k == 0u) continue;
                const uint32_t p = k >> sh_bits;
                if (p > prefix) ++my_sel;
                else if (p == prefix) {
                    if (exact || er < need) ++my_sel;
                    ++er;
                }
            }
        }
        uint32_t dst = off + block_excl_scan<kSelThreads>(my_sel, sh.scan, &tmp);
        {
            uint32_t er = eq_rank0;
            for (int i = i0; i < i1; ++i) {
                const uint32_t k = s_key[i];
                if (k == 0u) continue;
                const uint32_t p = k >> sh_bits;
                bool take = p > prefix;
                if (p == prefix) {
                    take = exact || er < need;
                    ++er;
                }
                if (take) {
                    int pos;
                    int64_t row;
                    cr.cand(s, c0 + i, c0, a.lp, pos, row);
                    if (dst < (uint32_t)K) {
                        st_agent(reinterpret_cast<uint32_t *>(out) + dst, (uint32_t)pos);
                        if (slots) st_agent(reinterpret_cast<uint32_t *>(slots) + dst, (uint32_t)row);
                    }
                    ++dst;
                }
            }
        }
    }
    if (chunk == G - 1)
        for (int j = (int)k_eff + tid; j < K; j += kSelThreads) {
            st_agent(reinterpret_cast<uint32_t *>(out) + j, 0xFFFFFFFFu);
            if (slots) st_agent(reinterpret_cast<uint32_t *>(slots) + j, 0xFFFFFFFFu);
        }

    // ---- leave the histograms zeroed for the next launch (the list path cleared its one
    //      above). Every histogram read happens before the count-exchange barrier; without
    //      that barrier (nothing to select) one more barrier separates the last reads from
    //      the clearing.
    if (!(k_eff > 0 && listn > 0)) {
        if (k_eff == 0) ok = group_barrier(&ss->count, G, a.err, nbar, a.spin_limit) && ok;
        for (int i = chunk * kSelThreads + tid; i < 3 * kHistBins; i += G * kSelThreads)
            st_agent(&ss->hist[0][0] + i, 0u);
    }

    // ---- leave. A wait that expired (the workgroups of the launch were not all resident at
    //      once, e.g. because other kernels held compute units) leaves the sequence's selection
    //      undefined: the last workgroup to leave, which every other one has left before with
    //      all its stores performed, then writes the defined failure result (every index -1;
    //      bit 0 of the error word is already set) and clears all three histograms, since a
    //      late workgroup may have added to them after the others cleared their slices. It
    //      also returns the record's counters and flag to zero.
    if (!ok && tid == 0) __hip_atomic_fetch_or(&ss->fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = fetch_add_agent(&ss->left, 1u);
        sh.res[0] = prev == (uint32_t)G - 1u ? 1u + (ld_agent(&ss->fail) != 0u ? 1u : 0u) : 0u;
    }
    __syncthreads();
    const uint32_t leave = sh.res[0];
    if (leave == 2u) {
        for (int j = tid; j < K; j += kSelThreads) {
            st_agent(reinterpret_cast<uint32_t *>(out) + j, 0xFFFFFFFFu);
            if (slots) st_agent(reinterpret_cast<uint32_t *>(slots) + j, 0xFFFFFFFFu);
        }
        for (int i = tid; i < 3 * kHistBins; i += kSelThreads) st_agent(&ss->hist[0][0] + i, 0u);
    }
    if (leave >= 1u && tid == 0) {
        st_agent(&ss->count, 0u);
        st_agent(&ss->left, 0u);
        st_agent(&ss->fail, 0u);
    }
}

template <int DIM, int HT, int KF, int MODE>
__global__ __launch_bounds__(kSelThreads, 1) void k_decode_select(SelectArgs a) {
    extern __shared__ uint32_t s_key[];  // [chunk] keys, then the chunk address table
    __shared__ SelShared sh;
    __shared__ u32x4 s_stage[kSelWaves][256];  // per-wave key-tile transpose area (4 KiB)
    int seq, chunk, G, ctx;
    if (!select_locate(
            a, [&](int c) { return sel_groups(ncand_of(MODE, c, a.lp, a.block_k), a.chunk); }, sh,
            seq, chunk, G, ctx))
        return;
    uint32_t nbar = 0;  // barriers passed (see group_barrier)
    select_run<DIM, HT, KF, MODE>(a, seq, chunk, G, ctx, a.sync + seq, nbar, true, s_key, sh,
                                  s_stage);
}

// Both stages of the hierarchical selection in one launch: the same workgroups score the block
// summaries and keep the block_k best blocks (ab: mode kBlocks, bf16 summaries), meet once more,
// then score the tokens of the kept blocks and keep the k best (ac: mode kCandidates). A
// sequence has the workgroups of its larger stage; the host picks the block stage's chunk so
// that this is the token stage. Each stage has its own record per sequence. The block list is
// written with agent-scope stores and read back with agent-scope loads.
template <int DIM, int HT, int KF>
__global__ __launch_bounds__(kSelThreads, 1) void k_decode_select_2l(SelectArgs ab, SelectArgs ac) {
    extern __shared__ uint32_t s_key[];  // the larger stage's keys and address table
    __shared__ SelShared sh;
    __shared__ u32x4 s_stage[kSelWaves][256];
    int seq, chunk, G, ctx;
    if (!select_locate(
            ac,
            [&](int c) {
                return max(sel_groups(ncand_of(kBlocks, c, ab.lp, ab.block_k), ab.chunk),
                           sel_groups(ncand_of(kCandidates, c, ac.lp, ac.block_k), ac.chunk));
            },
            sh, seq, chunk, G, ctx))
        return;
    uint32_t nb1 = 0;
    select_run<DIM, HT, kKeyBf16, kBlocks>(ab, seq, chunk, G, ctx, ab.sync + seq, nb1, true, s_key,
                                           sh, s_stage);
    // every workgroup of the sequence is past its block stage (the block list, or the failure
    // fill of its last workgroup, is complete) before any reads the list
    uint32_t nb2 = 0;
    const bool ok = group_barrier(&ac.sync[seq].count, (uint32_t)G, ac.err, nb2, ac.spin_limit);
    select_run<DIM, HT, KF, kCandidates>(ac, seq, chunk, G, ctx, ac.sync + seq, nb2, ok, s_key, sh,
                                         s_stage);
}

// ------------------------------------------------------------------ launchers
template <int DIM, int HT, int KF>
static hipError_t launch_score_t(const ScoreArgs &a, int rows, int64_t max_cols, hipStream_t st) {
    dim3 grid((unsigned)((max_cols + kScoreChunk - 1) / kScoreChunk), (unsigned)rows);
    hipLaunchKernelGGL((k_index_score<DIM, HT, KF>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int DIM, int MT, bool FP8>
static hipError_t launch_prefill_t(const ScoreArgs &a, hipStream_t st) {
    dim3 grid((unsigned)a.row_blocks, (unsigned)((a.ld + kPfTokens - 1) / kPfTokens));
    hipLaunchKernelGGL((k_prefill_score<DIM, MT, FP8>), grid, dim3(512), 0, st, a);
    return hipGetLastError();
}

template <int DIM, int KF>
static hipError_t launch_score_heads(const ScoreArgs &a, int heads, int rows, int64_t max_cols,
                                     hipStream_t st) {
    return heads <= 16 ? launch_score_t<DIM, 1, KF>(a, rows, max_cols, st)
                       : launch_score_t<DIM, 4, KF>(a, rows, max_cols, st);
}

template <int KF>
static hipError_t launch_score_kf(const ScoreArgs &a, int dim, int heads, int rows,
                                  int64_t max_cols, hipStream_t st) {
    return dim == 128 ? launch_score_heads<128, KF>(a, heads, rows, max_cols, st)
                      : launch_score_heads<64, KF>(a, heads, rows, max_cols, st);
}

hipError_t launch_index_score(const ScoreArgs &a, int dim, int heads, int key_fmt, int rows,
                              int64_t max_cols, hipStream_t st) {
    const bool fp8 = key_fmt == kKeyE4M3;
    // query rows grouped per sequence: dense GEMM (MXFP8 keys take the row-wise kernel, which
    // handles grouped rows too)
    if (a.q_indptr && key_fmt != kKeyMx) {
        if (a.row_blocks == 0) return hipSuccess;
        if (dim == 128) {
            if (heads <= 32) return fp8 ? launch_prefill_t<128, 1, true>(a, st) : launch_prefill_t<128, 1, false>(a, st);
            return fp8 ? launch_prefill_t<128, 2, true>(a, st) : launch_prefill_t<128, 2, false>(a, st);
        }
        if (heads <= 32) return fp8 ? launch_prefill_t<64, 1, true>(a, st) : launch_prefill_t<64, 1, false>(a, st);
        return fp8 ? launch_prefill_t<64, 2, true>(a, st) : launch_prefill_t<64, 2, false>(a, st);
    }
    if (key_fmt == kKeyMx) return launch_score_kf<kKeyMx>(a, dim, heads, rows, max_cols, st);
    if (fp8) return launch_score_kf<kKeyE4M3>(a, dim, heads, rows, max_cols, st);
    return launch_score_kf<kKeyBf16>(a, dim, heads, rows, max_cols, st);
}

template <int DIM, int HT, int KF, int MODE>
static void *select_kernel_ptr() {
    return reinterpret_cast<void *>(&k_decode_select<DIM, HT, KF, MODE>);
}

// pooled summaries (kBlocks) are bf16 whatever the key format; MXFP8 keys only take kTokens
template <int DIM, int HT>
static void *select_kernel_mode(int key_fmt, int mode) {
    if (mode == kBlocks) return select_kernel_ptr<DIM, HT, kKeyBf16, kBlocks>();
    if (key_fmt == kKeyMx) return mode == kTokens ? select_kernel_ptr<DIM, HT, kKeyMx, kTokens>() : nullptr;
    if (key_fmt == kKeyE4M3)
        return mode == kTokens ? select_kernel_ptr<DIM, HT, kKeyE4M3, kTokens>()
                               : select_kernel_ptr<DIM, HT, kKeyE4M3, kCandidates>();
    return mode == kTokens ? select_kernel_ptr<DIM, HT, kKeyBf16, kTokens>()
                           : select_kernel_ptr<DIM, HT, kKeyBf16, kCandidates>();
}

void *decode_select_kernel(int dim, int heads, int key_fmt, int mode) {
    const bool small = heads <= 16;
    if (dim == 128) return small ? select_kernel_mode<128, 1>(key_fmt, mode) : select_kernel_mode<128, 4>(key_fmt, mode);
    return small ? select_kernel_mode<64, 1>(key_fmt, mode) : select_kernel_mode<64, 4>(key_fmt, mode);
}

// Selection reuse: sequence s with reuse[s] >= 0 takes row reuse[s] (index set, and physical
// rows when given) once the selection of the other sequences is complete.
__global__ __launch_bounds__(256) void k_reuse_copy(const int32_t *reuse, int k, int32_t *idx,
                                                    int32_t *slots) {
    const int s = blockIdx.x, r = reuse[s];
    if (r < 0) return;
    for (int j = threadIdx.x; j < k; j += 256) {
        idx[(int64_t)s * k + j] = idx[(int64_t)r * k + j];
        if (slots) slots[(int64_t)s * k + j] = slots[(int64_t)r * k + j];
    }
}

hipError_t launch_reuse_copy(const int32_t *reuse, int num_seqs, int k, int32_t *idx,
                             int32_t *slots, hipStream_t st) {
    hipLaunchKernelGGL(k_reuse_copy, dim3((unsigned)num_seqs), dim3(256), 0, st, reuse, k, idx, slots);
    return hipGetLastError();
}

// the fused two-stage selection (bf16 or E4M3 keys; MXFP8 keys have no two-level path)
template <int DIM, int HT>
static void *select2l_kernel_fmt(int key_fmt) {
    // bf16 keys only: the block summaries are bf16 means of bf16 keys (the host rejects others)
    if (key_fmt == kKeyBf16) return reinterpret_cast<void *>(&k_decode_select_2l<DIM, HT, kKeyBf16>);
    return nullptr;
}

void *decode_select2l_kernel(int dim, int heads, int key_fmt) {
    const bool small = heads <= 16;
    if (dim == 128) return small ? select2l_kernel_fmt<128, 1>(key_fmt) : select2l_kernel_fmt<128, 4>(key_fmt);
    return small ? select2l_kernel_fmt<64, 1>(key_fmt) : select2l_kernel_fmt<64, 4>(key_fmt);
}

size_t decode_select_static_lds() { return sizeof(SelShared); }

size_t decode_select_dynamic_lds(int mode, int chunk, int lp) {
    const int t = chunk_table_entries(mode, chunk, lp);
    return 4 * ((size_t)chunk + t + (mode == kCandidates ? t : 0));
}

}  // namespace sa
