// Sparse attention over the gathered rows of the selected positions, gfx950.
//
// "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei
// Ascend CANN Architecture" §1 and §2.1 (the attention reads the KV precisely according to the
// selected indices); "Engineering Path for Day-0 Adaptation of Trillion-Scale Sparse Models on
// Domestic AI Accelerators" §3.1-§3.2 (non-contiguous access by index; block number + offset).
//
// One workgroup = one query row x one head group x one split of its index list. All heads
// share one KV row (MQA / MLA latent rows), so each gathered row is staged once in LDS and
// used by every wave:
//   S^T[tok][head] = K[tok][:] . Q[head][:]          (32x32x16 bf16 MFMA, K from LDS)
//   online softmax per head (lazy rescaling; a lane holds 16 tokens of one head)
//   O^T[d][head]  += V^T[d][tok] . P^T[tok][head]    (V^T fragments by transposing LDS reads)
// Splits write unnormalised partials that k_attn_merge combines.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTile = 32;          // gathered rows per iteration
// floats per lane row of the partial-score exchange: 32 scores + 4 padding, so that the
// 16-byte accesses of 16 consecutive lanes fall on distinct LDS banks
constexpr int kPartRow = 36;
constexpr float kRescale = 8.f;    // log2 growth tolerated before O is rescaled

// LDS row swizzle: 16-byte chunk c of staged row r lives at chunk c ^ swz(r). The XOR only
// touches the low three chunk bits, so a chunk stays inside its aligned group of 8. This
// choice keeps both the K-fragment reads (rows 0..31, one chunk each) and the transposing
// V reads (8 rows x 64 bytes) free of LDS bank conflicts with 1152-byte rows.
__device__ __forceinline__ int swz(int r) { return ((r << 1) & 6) ^ ((r >> 2) & 3); }

template <int DQK, int DV, bool SEPV, bool FP8>
struct AttnShape {
    static constexpr int KROW_G = FP8 ? DQK : 2 * DQK;  // global bytes per K row
    static constexpr int VROW_G = 2 * DV;                // (separate V rows are bf16)
    static constexpr int ROWB_K = 2 * DQK;               // LDS bytes per staged row (bf16)
    static constexpr int ROWB_V = 2 * DV;
    static constexpr int KBUF = kTile * ROWB_K;
    static constexpr int BUF = KBUF + (SEPV ? kTile * ROWB_V : 0);
    static constexpr int GCH_K = KROW_G / 16;            // 16-byte global chunks per K row
    static constexpr int GCH_V = SEPV ? VROW_G / 16 : 0;
    static constexpr int GCH = kTile * (GCH_K + GCH_V);  // global chunks per tile
};

// One workgroup = one quad of waves for one head group of 32 query heads. The four waves
// split the QK^T contraction over d (each adds a quarter of the k-steps; the partial scores are
// exchanged through LDS and summed in the same order by all four) and split the PV output
// over d_v (a quarter each). Each wave therefore holds a quarter of the query fragments and
// of the output accumulator, and two workgroups share a CU (two waves per SIMD) with about
// 60 KB of LDS each; running unsynchronised, the two overlap each other's MFMA, LDS and VALU
// phases. Gathered rows go global -> registers (one tile ahead) -> the single LDS tile.
template <int DQK, int DV, bool SEPV, bool FP8>
__global__ __launch_bounds__(256, 2) void k_sparse_attn(AttnArgs a) {
    using S = AttnShape<DQK, DV, SEPV, FP8>;
    constexpr int NT = 256;
    constexpr int NWV = 4;
    constexpr int NQ = 1;
    constexpr int KSP = DQK / 16 / 4;  // k-steps per wave
    constexpr int NDP = DV / 32 / 4;   // 32-wide d_v tiles per wave
    // staging: TPR threads per gathered row; thread (row, j) moves chunks j, j + TPR, ...
    constexpr int TPR = NT / kTile;
    constexpr int PER_K = (S::GCH_K + TPR - 1) / TPR;
    constexpr int PER_V = (S::GCH_V + TPR - 1) / TPR;
    constexpr int PER = PER_K + PER_V;
    static_assert(KSP * 64 == DQK && NDP * 128 == DV, "quarters of d and d_v");

    __shared__ __attribute__((aligned(16))) uint8_t stage[S::BUF];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // dynamic lds: [NWV][32][kPartRow] fp32 partial scores | [split_len] int32 slots |
    //              [split_len] fp32 logit bias (0, or -inf for an empty row) |
    //              [split_len] fp32 E4M3 row scale (0 for an empty row; E4M3 caches only)
    float *s_part = reinterpret_cast<float *>(lds);
    int32_t *s_slot = reinterpret_cast<int32_t *>(lds + NWV * 32 * kPartRow * 4);
    float *s_bias = reinterpret_cast<float *>(s_slot + a.split_len);
    float *s_sig = s_bias + a.split_len;

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int h = l >> 5, lm = l & 31;
    const int quad = 0, part = w;
    // block -> (row, head group, split); rows vary fastest so that with rows % 8 == 0 all
    // workgroups of one row land on the same XCD (blocks are dealt round-robin over XCDs)
    const int row = blockIdx.x % a.rows;
    const int hg = (blockIdx.x / a.rows) % a.hgroups;
    const int split = blockIdx.x / (a.rows * a.hgroups);
    int seq, qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int32_t *pt = a.page_table + (int64_t)seq * a.pages_per_seq;
    const int32_t *idx = a.idx + (int64_t)row * a.k;
    const int j0 = split * a.split_len;
    const int j1 = min(a.k, j0 + a.split_len);
    const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;
    const int P = 1 << a.lp;

    // ---- slot and flag of every selected row of this split (the loop below then issues no
    //      dependent global loads)
    for (int j = tid; j < ntiles * kTile; j += NT) {
        int32_t slot = -1;
        if (j0 + j < j1) {
            const int e = idx[j0 + j];
            if (e >= 0) slot = pt[e >> a.lp] * P + (e & (P - 1));
        }
        s_slot[j] = slot;
        s_bias[j] = slot < 0 ? -__builtin_inff() : 0.f;
        if (FP8) s_sig[j] = slot < 0 ? 0.f : a.kv_scale[slot];
    }

    // query fragments (B operand of S^T = K Q^T): head `head`, d = 16 s + 8 h + e for this
    // wave's k-steps s in [part * KSP, part * KSP + KSP)
    const int head = 32 * (NQ * hg + quad) + lm;
    u32x4 qf[KSP];
    {
        const uint16_t *qr = a.q + ((int64_t)row * a.heads_q + head) * DQK + 8 * h;
#pragma unroll
        for (int s = 0; s < KSP; ++s)
            qf[s] = head < a.heads_q ? ldg16(qr + 16 * (part * KSP + s)) : u32x4{0u, 0u, 0u, 0u};
    }
    // Query fragments and the slot table complete here, so that inside the tile loop the only
    // vector-memory loads in flight are the staging loads of the next tile, which nothing in
    // the loop body before the staging store waits for.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // slot table ready

    // ---- gather: global chunk i of the tile -> registers -> swizzled LDS chunk(s)
    u32x4 stg[PER];
    const int srow = tid / TPR, sj = tid % TPR;
    // An empty slot (or a tile past the end) stages the workspace's zero row: its logit gets
    // the -inf bias and its V row contributes 0 * 0. Loads are unconditional wherever a row
    // divides evenly among its threads.
    auto load = [&](int t, u32x4 (&v)[PER]) {
        const int32_t slot = t < ntiles ? s_slot[t * kTile + srow] : -1;
        const uint8_t *kr = slot < 0 ? a.zero_row : a.kc + (int64_t)slot * S::KROW_G;
        const uint8_t *vr = SEPV ? (slot < 0 ? a.zero_row : a.vc + (int64_t)slot * S::VROW_G)
                                 : nullptr;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool isv = i >= PER_K;
            const int col = sj + TPR * (isv ? i - PER_K : i);
            const int gch = isv ? S::GCH_V : S::GCH_K;
            const bool even = (isv ? S::GCH_V : S::GCH_K) % TPR == 0;
            v[i] = (even || col < gch) ? ldg16((isv ? vr : kr) + 16 * col) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](const u32x4 (&v)[PER], uint8_t *buf) {
        const int r = srow, sw = swz(srow);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool isv = i >= PER_K;
            const int col = sj + TPR * (isv ? i - PER_K : i);
            if (col < (isv ? S::GCH_V : S::GCH_K)) {
                uint8_t *rowp = isv ? buf + S::KBUF + r * S::ROWB_V : buf + r * S::ROWB_K;
                if (FP8) {
                    // 16 codes -> 16 bf16 (exact); the row scale is applied to logits and P
                    const u32x2 q0 = e4m3x4_to_bf16(v[i][0]), q1 = e4m3x4_to_bf16(v[i][1]);
                    const u32x2 q2 = e4m3x4_to_bf16(v[i][2]), q3 = e4m3x4_to_bf16(v[i][3]);
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col) ^ sw)) =
                        u32x4{q0[0], q0[1], q1[0], q1[1]};
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col + 1) ^ sw)) =
                        u32x4{q2[0], q2[1], q3[0], q3[1]};
                } else {
                    *reinterpret_cast<u32x4 *>(rowp + 16 * (col ^ sw)) = v[i];
                }
            }
        }
    };

    f32x16 o[NDP];
#pragma unroll
    for (int n = 0; n < NDP; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;

    // prologue: tile 0 into LDS, tile 1 into registers
    if (ntiles > 0) {
        load(0, stg);
        store(stg, stage);
        load(1, stg);
        lds_barrier();
    }
    const int g = l >> 4, jj = l & 15;
    // tile t is in `stage`; the registers hold tile t+1, written into `stage` once every wave
    // is done with tile t, and then receive the loads of tile t+2
    for (int t = 0; t < ntiles; ++t) {
        const uint8_t *cur = stage;
        const uint8_t *vb = SEPV ? cur + S::KBUF : cur;
        constexpr int VROWB = SEPV ? S::ROWB_V : S::ROWB_K;
        // ---- partial S^T = K Q^T over this wave's quarter of d
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        const uint8_t *krow = cur + lm * S::ROWB_K;
        const int sw = swz(lm);
#pragma unroll
        for (int s = 0; s < KSP; ++s) {
            const int c = 2 * (part * KSP + s) + h;
            const u32x4 kf = *reinterpret_cast<const u32x4 *>(krow + 16 * (c ^ sw));
            sacc = mfma32x32x16(kf, qf[s], sacc);
        }
        float *mine_s = s_part + (w * 32 + lm) * kPartRow + 16 * h;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4 *>(mine_s + 4 * q4) =
                f32x4{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
        lds_barrier();
        // ---- full scores: the quad's four partials, all read back from LDS and summed in
        //      the same order by every wave (identical scores in all four); logits in the log2
        //      domain as one FMA with the row's bias (-inf for an empty row, whose staged K
        //      row is zero)
        const float *sig = s_sig + t * kTile;
        const float *bia = s_bias + t * kTile;
        float m_tile = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 sum = *reinterpret_cast<const f32x4 *>(s_part + ((quad * 4) * 32 + lm) * kPartRow + 16 * h + 4 * j);
#pragma unroll
            for (int p = 1; p < 4; ++p)
                sum += *reinterpret_cast<const f32x4 *>(
                    s_part + ((quad * 4 + p) * 32 + lm) * kPartRow + 16 * h + 4 * j);
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(bia + 8 * j + 4 * h);
            f32x4 sv = {1.f, 1.f, 1.f, 1.f};
            if (FP8) sv = *reinterpret_cast<const f32x4 *>(sig + 8 * j + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                sacc[r] = fmaf(sum[i], FP8 ? a.scale_log2 * sv[i] : a.scale_log2, bv[i]);
                m_tile = fmaxf(m_tile, sacc[r]);
            }
        }
        m_tile = max_xor32(m_tile);
        const bool grow = m_tile > m_run + kRescale;
        if (__any(grow)) {
            const float m_new = grow ? m_tile : m_run;
            // alpha = 0 when m_run = -inf (nothing accumulated yet)
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < NDP; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[n][r] *= alpha;
            m_run = m_new;
        }
        // while m_run is -inf every logit seen so far was -inf: subtracting 0 keeps p = 0
        const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
        u32x4 pb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t pk[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float pp[2];
#pragma unroll
                for (int e1 = 0; e1 < 2; ++e1) {
                    const int r = 8 * u + 2 * e2 + e1;
                    const float p = __builtin_amdgcn_exp2f(sacc[r] - m_use);
                    l_run += p;
                    pp[e1] = FP8 ? p * sig[8 * (r >> 2) + 4 * h + (r & 3)] : p;
                }
                pk[e2] = pack_bf16x2(pp[0], pp[1]);
            }
            pb[u] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        }
        // ---- O^T += V^T P^T over this wave's quarter of d_v: two 16-token k-steps
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ra = 16 * u + 4 * (g >> 1) + (jj >> 2), rb = ra + 8;
            const uint8_t *va = vb + ra * VROWB, *vbp = vb + rb * VROWB;
            const int swa = swz(ra), swb = swz(rb);
            const int byte_in = 8 * (jj & 1);
#pragma unroll
            for (int n = 0; n < NDP; ++n) {
                const int c = 4 * (part * NDP + n) + 2 * (g & 1) + ((jj & 3) >> 1);
                const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SA_LDS i16x4 *)(va + 16 * (c ^ swa) + byte_in));
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SA_LDS i16x4 *)(vbp + 16 * (c ^ swb) + byte_in));
                const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
                const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
                o[n] = mfma32x32x16(u32x4{w0[0], w0[1], w1[0], w1[1]}, pb[u], o[n]);
            }
        }
        // ---- stage tile t+1 (loaded during this tile) and start the loads of tile t+2
        lds_barrier();  // every wave is done reading tile t
        if (t + 1 < ntiles) store(stg, stage);
        load(t + 2, stg);
        lds_barrier();
    }

    // ---- epilogue: this wave owns d_v tiles [part * NDP, part * NDP + NDP) of head `head`
    const float l_tot = sum_xor32(l_run);
    if (head >= a.heads_q) return;
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * DV;
#pragma unroll
        for (int n = 0; n < NDP; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * (part * NDP + n) + 8 * j + 4 * h;
                u32x2 v = {pack_bf16x2(o[n][4 * j] * inv, o[n][4 * j + 1] * inv),
                           pack_bf16x2(o[n][4 * j + 2] * inv, o[n][4 * j + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + d) = v;
            }
    } else {
        // partial of this split, normalised by its own sum, in bf16 (the merge weights carry
        // the sums); empty splits write zeros and l = 0
        const int64_t ph = ((int64_t)row * a.splits + split) * a.heads_q + head;
        uint16_t *orow = a.part_o + ph * DV;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int n = 0; n < NDP; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * (part * NDP + n) + 8 * j + 4 * h;
                u32x2 v = {pack_bf16x2(o[n][4 * j] * inv, o[n][4 * j + 1] * inv),
                           pack_bf16x2(o[n][4 * j + 2] * inv, o[n][4 * j + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + d) = v;
            }
        if (h == 0 && part == 0) {
            a.part_ml[2 * ph] = m_run;
            a.part_ml[2 * ph + 1] = l_tot;
        }
    }
}

// Combine split partials: o = sum_s w_s o_s / sum_s w_s with w_s = 2^(m_s - M) l_s and o_s the
// split's own normalised output. Grid: rows x ceil(heads/4); 256 threads = 4 heads x 64
// threads x (DV/64) entries.
template <int DV>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
    constexpr int PER = DV / 64;      // output entries per thread
    constexpr int WPS = PER / 2;      // 32-bit words (bf16 pairs) per split and thread
    constexpr int BATCH = 8;          // splits whose loads are in flight together
    static_assert(PER % 2 == 0, "whole bf16 pairs per thread");
    const int row = blockIdx.x;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (head >= a.heads_q) return;
    const int d0 = (threadIdx.x & 63) * PER;
    const int64_t ph0 = (int64_t)row * a.splits * a.heads_q + head;  // split s: ph0 + s * heads_q
    // online combination in split order: running max M, sum L and output (rescaled when M
    // grows); splits without selected rows (l = 0) are skipped
    float M = -__builtin_inff(), L = 0.f, acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < a.splits; s0 += BATCH) {
        float2 ml[BATCH];
        uint32_t v[BATCH][WPS];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            ml[u] = float2{-__builtin_inff(), 0.f};
            if (s0 + u < a.splits) {
                const int64_t ph = ph0 + (int64_t)(s0 + u) * a.heads_q;
                ml[u] = *reinterpret_cast<const float2 *>(a.part_ml + 2 * ph);
                const uint32_t *po = reinterpret_cast<const uint32_t *>(a.part_o + ph * DV + d0);
#pragma unroll
                for (int x = 0; x < WPS; ++x) v[u][x] = po[x];
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (!(ml[u].y > 0.f)) continue;
            const float mn = fmaxf(M, ml[u].x);
            const float c = __builtin_amdgcn_exp2f(M - mn);  // 0 while nothing is accumulated
            const float wgt = __builtin_amdgcn_exp2f(ml[u].x - mn) * ml[u].y;
            L = fmaf(L, c, wgt);
#pragma unroll
            for (int x = 0; x < WPS; ++x) {
                acc[2 * x] = fmaf(acc[2 * x], c, wgt * bf16_lo(v[u][x]));
                acc[2 * x + 1] = fmaf(acc[2 * x + 1], c, wgt * bf16_hi(v[u][x]));
            }
            M = mn;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * DV + d0;
#pragma unroll
    for (int e = 0; e < PER; e += 2)
        *reinterpret_cast<uint32_t *>(orow + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
}

template <int DQK, int DV, bool SEPV, bool FP8>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
    const size_t lds = (size_t)4 * 32 * kPartRow * 4 + (size_t)a.split_len * (FP8 ? 12 : 8);
    auto kern = k_sparse_attn<DQK, DV, SEPV, FP8>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.rows * a.splits * a.hgroups)), dim3(256), lds, st,
                       a);
    e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(k_attn_merge<DV>, dim3((unsigned)a.rows, (unsigned)((a.heads_q + 3) / 4)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs &a, int dqk, int dv, bool sep_v, bool fp8,
                              hipStream_t st) {
    if (dqk == 576 && dv == 512 && !sep_v)
        return fp8 ? launch_attn_t<576, 512, false, true>(a, st)
                   : launch_attn_t<576, 512, false, false>(a, st);
    if (dqk == 128 && dv == 128 && !fp8)
        return sep_v ? launch_attn_t<128, 128, true, false>(a, st)
                     : launch_attn_t<128, 128, false, false>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace sa
