// Sparse attention over the gathered rows of the selected positions, gfx950.
//
// "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei
// Ascend CANN Architecture" §1 and §2.1 (the attention reads only the KV rows the index set
// names); "Engineering Path for Day-0 Adaptation of Trillion-Scale Sparse Models on Domestic
// AI Accelerators" §3.1-§3.2 (non-contiguous access by index; block number + offset).
//
// All query heads share one KV row (MQA / MLA latent rows), so each gathered row is staged
// once in LDS and used by every wave of the workgroup (see k_sparse_attn_pairs). Index sets
// split over several workgroups publish normalised partials that k_attn_merge combines.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTile = 32;          // gathered rows per iteration
constexpr float kRescale = 8.f;    // log2 growth tolerated before O is rescaled

// LDS row swizzle: 16-byte chunk c of staged row r lives at chunk c ^ swz(r). The XOR only
// touches the low three chunk bits, so a chunk stays inside its aligned group of 8. With
// 1152-byte rows it keeps three access patterns free of LDS bank conflicts: the staging stores
// (16 consecutive chunks of a row), the K-fragment reads (16 rows, one chunk each) and the
// transposing V reads, where 32 lanes read rows {4g, 4g+1, 16+4g, 16+4g+1} (or the other four
// of the group) x 32 bytes for two lane groups g at once.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r >> 2) & 4); }

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

// One workgroup = 8 waves for one query row, a group of 64 query heads and one split of its
// index list; one workgroup per CU. Wave w forms pair w / 2 (16 heads) with its partner w ^ 1:
//   S^T[row][head] = K[row][:] . Q[head][:]   (16x16x32 bf16 MFMA; each wave of a pair adds one
//                                              half of d, the halves are exchanged through LDS)
//   online softmax per head (a lane holds 8 rows of one head)
//   O^T[d][head] += V^T[d][row] . P^T[row][head]  (each wave of a pair owns one half of d_v;
//                                                  V^T fragments by transposing LDS reads)
// Gathered rows go global -> registers (one tile ahead) -> one of two LDS tiles, so the store
// of the next tile overlaps nothing but is covered by a whole tile of loads.
constexpr int kPairHeads = 64;

// FP8 rows carry one scale per row, or with T128 one scale per 128-entry tile ([CANN] §3:
// per-token-head-tile FP8 KV). Codes are widened to bf16 exactly either way; a row scale
// multiplies the logits and P, tile scales multiply the per-tile partial dot products (QK) and
// one copy of P per tile of d_v (PV).
template <int DQK, int DV, bool SEPV, bool FP8, bool T128 = false>
__global__ __launch_bounds__(512, 1) void k_sparse_attn_pairs(AttnArgs a) {
    using S = AttnShape<DQK, DV, SEPV, FP8>;
    constexpr bool ROWSC = FP8 && !T128;                 // one scale per row
    constexpr int NSC = T128 ? (DQK + 127) / 128 : 1;    // scales per row
    static_assert(!T128 || (FP8 && !SEPV && DV == 512), "tile scales: latent E4M3 rows");
    constexpr int NT = 512;
    constexpr int KH = DQK / 32 / 2;    // k-steps per wave (half of d)
    constexpr int DT = DV / 16 / 2;     // 16-wide d_v tiles per wave (half of d_v)
    static_assert(KH * 64 == DQK && DT * 32 == DV, "halves of d and d_v");
    constexpr int TPR = NT / kTile;     // staging threads per gathered row
    constexpr int PER_K = (S::GCH_K + TPR - 1) / TPR;
    constexpr int PER_V = (S::GCH_V + TPR - 1) / TPR;
    constexpr int PER = PER_K + PER_V;
    constexpr int VROWB = SEPV ? S::ROWB_V : S::ROWB_K;

    __shared__ __attribute__((aligned(16))) uint8_t stage[2][S::BUF];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // dynamic lds: [4 pairs][2 halves][2][64 lanes] f32x4 partial scores | [split_len] int32
    // slots | [split_len] fp32 logit bias (0 or -inf) | E4M3 scales (E4M3 only): [split_len]
    // per row, or [NSC][split_len] per tile
    f32x4 *s_x = reinterpret_cast<f32x4 *>(lds);
    int32_t *s_slot = reinterpret_cast<int32_t *>(lds + 4 * 2 * 2 * 64 * 16);
    float *s_bias = reinterpret_cast<float *>(s_slot + a.split_len);
    float *s_sig = s_bias + a.split_len;

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int pair = w >> 1, half = w & 1, g = l >> 4, L = l & 15;
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

    // ---- slot, bias and scale of every selected row of this split
    for (int j = tid; j < ntiles * kTile; j += NT) {
        int32_t slot = -1;
        if (j0 + j < j1) {
            if (a.slots) {
                slot = a.slots[(int64_t)row * a.k + j0 + j];
            } else {
                const int e = idx[j0 + j];
                if (e >= 0) slot = pt[e >> a.lp] * P + (e & (P - 1));
            }
        }
        s_slot[j] = slot;
        s_bias[j] = slot < 0 ? -__builtin_inff() : 0.f;
        if (ROWSC) s_sig[j] = slot < 0 ? 0.f : a.kv_scale[slot];
        if (T128)
#pragma unroll
            for (int c = 0; c < NSC; ++c)
                s_sig[c * a.split_len + j] = slot < 0 ? 0.f : a.kv_scale[(int64_t)slot * NSC + c];
    }
    __syncthreads();  // the slot table is complete: load(0) reads rows written by other threads
    // query fragments (B operand of S^T = K Q^T): head L of the pair, d = 32 s + 8 g + e for
    // this wave's half of the k-steps. A lane past the last head reads head 0 (its column of
    // scores stays its own and is never stored), so no load sits behind a branch. They are
    // issued together with the first tile's rows and complete before its store.
    const int head = kPairHeads * hg + 16 * pair + L;
    const bool live = head < a.heads_q;
    u32x4 qf[KH];
    {
        const uint16_t *qr = a.q + ((int64_t)row * a.heads_q + (live ? head : 0)) * DQK + 8 * g;
#pragma unroll
        for (int s = 0; s < KH; ++s) qf[s] = ldg16(qr + 32 * (half * KH + s));
    }

    // ---- gather: thread (row srow, j = sj) moves global chunks j, j + TPR, ... of its row
    u32x4 stg[PER];
    const int srow = tid / TPR, sj = tid % TPR;
    auto load = [&](int t) {
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
            stg[i] = (even || col < gch) ? ldg16((isv ? vr : kr) + 16 * col) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](uint8_t *buf) {
        const int r = srow, sw = swz(srow);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const bool isv = i >= PER_K;
            const int col = sj + TPR * (isv ? i - PER_K : i);
            if (col < (isv ? S::GCH_V : S::GCH_K)) {
                uint8_t *rowp = isv ? buf + S::KBUF + r * S::ROWB_V : buf + r * S::ROWB_K;
                if (FP8) {
                    // 16 codes -> 16 bf16 (exact); the row scale is applied to logits and P
                    const u32x2 q0 = e4m3x4_to_bf16(stg[i][0]), q1 = e4m3x4_to_bf16(stg[i][1]);
                    const u32x2 q2 = e4m3x4_to_bf16(stg[i][2]), q3 = e4m3x4_to_bf16(stg[i][3]);
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col) ^ sw)) =
                        u32x4{q0[0], q0[1], q1[0], q1[1]};
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col + 1) ^ sw)) =
                        u32x4{q2[0], q2[1], q3[0], q3[1]};
                } else {
                    *reinterpret_cast<u32x4 *>(rowp + 16 * (col ^ sw)) = stg[i];
                }
            }
        }
    };

    f32x4 o[DT];
#pragma unroll
    for (int n = 0; n < DT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;

    if (ntiles > 0) {
        load(0);
        store(stage[0]);
        load(1);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const uint8_t *kb = stage[t & 1];
        const uint8_t *vb = SEPV ? kb + S::KBUF : kb;
        // the other buffer held tile t - 1, whose reads ended before the last barrier
        if (t + 1 < ntiles) store(stage[(t + 1) & 1]);
        load(t + 2);
        // ---- partial S^T over this wave's half of d: two 16-row M tiles
        f32x4 sa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (!T128) {
#pragma unroll
            for (int s = 0; s < KH; ++s)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int r = 16 * mt + L;
                    const u32x4 kf = *reinterpret_cast<const u32x4 *>(
                        kb + r * S::ROWB_K + 16 * ((4 * (half * KH + s) + g) ^ swz(r)));
                    sa[mt] = mfma16x16x32(kf, qf[s], sa[mt]);
                }
        } else {
            // one accumulator per 128-entry tile that this half of d touches (k-step s of the
            // row covers d = 32 s .. 32 s + 31, so tile s / 4); the tile's scales of the lane's
            // rows (16 mt + 4 g + i) multiply it before the halves are exchanged
            auto qk_half = [&](auto hc) {
                constexpr int H = decltype(hc)::value;
                constexpr int T0 = (H * KH) / 4, NTL = (H * KH + KH - 1) / 4 - T0 + 1;
                f32x4 acc[NTL][2];
#pragma unroll
                for (int tl = 0; tl < NTL; ++tl)
                    acc[tl][0] = acc[tl][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KH; ++s)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const int r = 16 * mt + L;
                        const u32x4 kf = *reinterpret_cast<const u32x4 *>(
                            kb + r * S::ROWB_K + 16 * ((4 * (H * KH + s) + g) ^ swz(r)));
                        const int tl = (H * KH + s) / 4 - T0;
                        acc[tl][mt] = mfma16x16x32(kf, qf[s], acc[tl][mt]);
                    }
#pragma unroll
                for (int tl = 0; tl < NTL; ++tl)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const f32x4 sg = *reinterpret_cast<const f32x4 *>(
                            s_sig + (T0 + tl) * a.split_len + t * kTile + 16 * mt + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sa[mt][i] = fmaf(acc[tl][mt][i], sg[i], sa[mt][i]);
                    }
            };
            if (half == 0) qk_half(std::integral_constant<int, 0>{});
            else qk_half(std::integral_constant<int, 1>{});
        }
        // ---- exchange halves with the partner wave (float addition commutes, so both waves
        //      obtain the same sums)
        f32x4 *xo = s_x + ((pair * 2 + half) * 2) * 64 + l;
        xo[0] = sa[0];
        xo[64] = sa[1];
        lds_barrier();
        const f32x4 *xp = s_x + ((pair * 2 + (half ^ 1)) * 2) * 64 + l;
        const f32x4 sum0 = sa[0] + xp[0], sum1 = sa[1] + xp[64];
        // ---- logits in the log2 domain: rows 16 mt + 4 g + i of head L
        const float *bia = s_bias + t * kTile + 4 * g;
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bia);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bia + 16);
        f32x4 sg0 = {1.f, 1.f, 1.f, 1.f}, sg1 = {1.f, 1.f, 1.f, 1.f};
        if (ROWSC) {
            sg0 = *reinterpret_cast<const f32x4 *>(s_sig + t * kTile + 4 * g);
            sg1 = *reinterpret_cast<const f32x4 *>(s_sig + t * kTile + 4 * g + 16);
        }
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = fmaf(sum0[i], ROWSC ? a.scale_log2 * sg0[i] : a.scale_log2, b0[i]);
            x[4 + i] = fmaf(sum1[i], ROWSC ? a.scale_log2 * sg1[i] : a.scale_log2, b1[i]);
        }
        float m_tile = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        m_tile = fmaxf(m_tile, __shfl_xor(m_tile, 16, 64));
        m_tile = max_xor32(m_tile);
        const bool grow = m_tile > m_run + kRescale;
        if (__any(grow)) {
            const float m_new = grow ? m_tile : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < DT; ++n) o[n] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
            l_run += p[e];
        }
        if (ROWSC) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] *= sg0[i];
                p[4 + i] *= sg1[i];
            }
        }
        // P^T B operand: k = 8 g + e <-> the lane's own rows, in the order of the V reads below:
        // e = 0..3 rows 4g, 4g+1, 16+4g, 16+4g+1; e = 4..7 the same plus 2. With tile scales,
        // one operand per 128-entry tile of this wave's half of d_v, P scaled by that tile's
        // scales of the lane's rows.
        constexpr int NPB = T128 ? (DV / 2) / 128 : 1;
        u32x4 pbs[NPB];
#pragma unroll
        for (int tt = 0; tt < NPB; ++tt) {
            f32x4 s0 = {1.f, 1.f, 1.f, 1.f}, s1 = {1.f, 1.f, 1.f, 1.f};
            if (T128) {
                const float *sp = s_sig + (half * NPB + tt) * a.split_len + t * kTile + 4 * g;
                s0 = *reinterpret_cast<const f32x4 *>(sp);
                s1 = *reinterpret_cast<const f32x4 *>(sp + 16);
            }
            pbs[tt] = u32x4{pack_bf16x2(p[0] * s0[0], p[1] * s0[1]), pack_bf16x2(p[4] * s1[0], p[5] * s1[1]),
                            pack_bf16x2(p[2] * s0[2], p[3] * s0[3]), pack_bf16x2(p[6] * s1[2], p[7] * s1[3])};
        }
        // ---- O^T += V^T P^T over this wave's half of d_v. Transposing reads: input lane j of
        //      group g loads columns [4 (j % 4), +4) of row R(j / 4), with R(q) = 4 g + (q & 1)
        //      + 16 (q >> 1) (+ 2 for the second read); output lane L then holds column L of
        //      rows R(0) .. R(3).
        const int q = L >> 2;
        const int vr1 = 4 * g + (q & 1) + 16 * (q >> 1), vr2 = vr1 + 2;
        const uint8_t *va = vb + vr1 * VROWB, *vbp = vb + vr2 * VROWB;
        const int sw1 = swz(vr1), sw2 = swz(vr2);
        const int byte_in = 8 * ((L & 3) & 1);
#pragma unroll
        for (int n = 0; n < DT; ++n) {
            const int c = (half * (DV / 2) + 16 * n) / 8 + ((L & 3) >> 1);
            const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SA_LDS i16x4 *)(va + 16 * (c ^ sw1) + byte_in));
            const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SA_LDS i16x4 *)(vbp + 16 * (c ^ sw2) + byte_in));
            const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
            o[n] = mfma16x16x32(u32x4{w0[0], w0[1], w1[0], w1[1]}, pbs[(16 * n * NPB) / (DV / 2)], o[n]);
        }
        lds_barrier();  // tile t fully read; tile t + 1 stored
    }

    // ---- epilogue: lane L of group g holds d_v = half * DV / 2 + 16 n + 4 g + i of head L
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot = sum_xor32(l_tot);
    if (!live) return;
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * DV;
#pragma unroll
        for (int n = 0; n < DT; ++n) {
            const int d = half * (DV / 2) + 16 * n + 4 * g;
            *reinterpret_cast<u32x2 *>(orow + d) =
                u32x2{pack_bf16x2(o[n][0] * inv, o[n][1] * inv), pack_bf16x2(o[n][2] * inv, o[n][3] * inv)};
        }
    } else {
        const int64_t ph = ((int64_t)row * a.splits + split) * a.heads_q + head;
        uint16_t *orow = a.part_o + ph * DV;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int n = 0; n < DT; ++n) {
            const int d = half * (DV / 2) + 16 * n + 4 * g;
            *reinterpret_cast<u32x2 *>(orow + d) =
                u32x2{pack_bf16x2(o[n][0] * inv, o[n][1] * inv), pack_bf16x2(o[n][2] * inv, o[n][3] * inv)};
        }
        if (g == 0 && half == 0) {
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

// ================================================== latent rows, many query heads per workgroup
// bf16 latent rows (576 entries: the first 512 are V) and up to 128 query heads sharing them
// (MLA-style decode and prefill; [CANN] §1 and §2.1). One workgroup of 8 waves per (query row,
// head group, split of its index set). Each wave owns 16 heads with the whole 576-wide
// contraction, so a staged row serves all the workgroup's heads and no partial score crosses
// waves:
//   S^T[row][head] = K[row][:] . Q[head][:]       (16x16x32 bf16 MFMA, 2 x 18 per 32-row tile)
//   online softmax per head                        (a lane holds 8 rows of one head)
//   O^T[d][head] += V^T[d][row] . P^T[row][head]  (32 MFMAs per tile, V^T by transposing reads)
// Two tile-phase layouts (template T):
//   T = 1: 8 waves x 16 heads = 128 heads; every wave computes every tile. One head group.
//   T = 2: 4 groups of 16 heads x 2 phases = 64 heads; phase p computes the tiles t = p mod 2,
//          and at the end phase 1 hands its (max, sum, output) to phase 0 through LDS. With more
//          than 64 heads a row has two head groups; they gather the same rows, the second from
//          the L2 of the XCD they share.
// T = 2 halves what a split publishes for the merge (64 heads instead of 128), which is what
// decode, with few rows and many splits, pays most for.
// Two waves per SIMD keep the 16x16x32 MFMA at its full rate. A wave's query fragments (72
// registers) and output accumulators (128) take most of its 256, so addresses are rebuilt per
// tile and LDS reads run only a few fragments ahead of their MFMAs.
// Rows move from HBM straight into LDS (global_load_lds_dwordx4) through a ring of tiles of 32
// rows (T = 1: four, three in flight while one is computed; T = 2: four, one step of two tiles
// in flight while the other is computed), and the copies use no registers. With T = 2 a step's
// copies are issued as soon as a barrier shows the slots they overwrite free, before the wait
// for the step about to be computed, so that its single step ahead never drains. Every wave
// issues the same number of 1 KiB copies per step, so every wave waits for an exact count.
//
// Index sets split over several workgroups (few query rows, as in decode) are merged inside the
// same launch: each split publishes its output normalised by its own sum (bf16) with its
// (max, sum) per head through agent-scope stores, the splits of a (row, head group) meet at a
// barrier, and then split s merges the units [s U / S, (s + 1) U / S) of all splits, in split
// order (the result does not depend on timing). This needs every split resident at once: the
// host only chooses it when the grid fits the device's resident capacity. Workgroup b runs on
// XCD b mod 8 (round-robin dispatch), so the workgroups of a row are given indices of one
// residue mod 8: they share that XCD's L2.
constexpr int kLatQK = 576, kLatV = 512;
constexpr int kLatRowB = 2 * kLatQK;          // bytes per staged row
constexpr int kLatTileB = kTile * kLatRowB;   // 36864 bytes per tile
constexpr int kLatWaves = 8;
constexpr int kLatThreads = 64 * kLatWaves;
constexpr int kLatKS = kLatQK / 32;           // 18 k-steps of 32 entries
constexpr int kLatDT = kLatV / 16;            // 32 d_v tiles of 16 entries
static_assert(kLatTileB == 36 * 1024, "36 one-KiB copies per tile");

// Workgroup b -> (query row, head group, split). A row has U = hgroups * splits workgroups. With
// xcd_align the U workgroups of row r get indices of one residue mod 8 (r mod 8), so they run on
// one XCD: the head groups of a split then share that XCD's L2 for the gathered rows, and the
// merge reads partials written on the same XCD. Padding workgroups (row >= rows) exit at once.
__device__ __forceinline__ void lat_unit_of(int b, const AttnArgs &a, int &r, int &hgi,
                                            int &split) {
    const int U = a.hgroups * a.splits;
    int u;
    if (a.xcd_align) {
        const int local = b >> 3;
        r = 8 * (local / U) + (b & 7);
        u = local % U;
    } else {
        r = b / U;
        u = b % U;
    }
    hgi = u % a.hgroups;
    split = u / a.hgroups;
}

__host__ __device__ inline int lat_grid(int rows, int units, int xcd_align) {
    return xcd_align ? 8 * units * ((rows + 7) / 8) : rows * units;
}

// A value the compiler may not take apart (so that it keeps a base register and folds
// constants into instruction offsets instead of hoisting one register per address).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// The merge of a (row, head group): units [u0, u1) of every split's partial block combined in
// split order (running max and rescale, as an online softmax over the splits), written to the
// output with agent-scope stores. MU units per thread and MS splits have their loads in flight
// together (MU * MS <= 16 keeps the loads' registers below the kernel's budget).
template <int HPW, int MU, int MS>
__device__ __forceinline__ void lat_merge_units(const AttnArgs &a, int row, int hgi, int64_t grp,
                                                int64_t blk_elems, int u0, int u1) {
    const int tid = threadIdx.x;
    for (int ub = u0 + tid; ub < u1; ub += MU * kLatThreads) {
        int hl[MU];
        bool on[MU];
        float M[MU], Lsum[MU], acc[MU][4];
#pragma unroll
        for (int i = 0; i < MU; ++i) {
            const int u = ub + i * kLatThreads;
            hl[i] = 16 * (u >> 11) + (u & 15);  // head inside the group
            on[i] = u < u1 && HPW * hgi + hl[i] < a.heads_q;
            if (!on[i]) hl[i] = 0;  // (loads stay in bounds; results unused)
            M[i] = -__builtin_inff();
            Lsum[i] = 0.f;
            acc[i][0] = acc[i][1] = acc[i][2] = acc[i][3] = 0.f;
        }
        for (int s0 = 0; s0 < a.splits; s0 += MS) {
            uint64_t ml[MU][MS], v[MU][MS];
#pragma unroll
            for (int x = 0; x < MS; ++x) {
                const int64_t gs = grp * a.splits + min(s0 + x, a.splits - 1);
#pragma unroll
                for (int i = 0; i < MU; ++i) {
                    const int u = on[i] ? ub + i * kLatThreads : u0;
                    ml[i][x] = ld_agent_u64(a.part_ml + 2 * (gs * HPW + hl[i]));
                    v[i][x] = ld_agent_u64(a.part_o + gs * blk_elems + 4 * (int64_t)u);
                }
            }
#pragma unroll
            for (int i = 0; i < MU; ++i)
#pragma unroll
                for (int x = 0; x < MS; ++x) {
                    const float ms = __uint_as_float((uint32_t)ml[i][x]);
                    const float ls = __uint_as_float((uint32_t)(ml[i][x] >> 32));
                    if (s0 + x >= a.splits || !(ls > 0.f)) continue;
                    const float mn = fmaxf(M[i], ms);
                    const float c = __builtin_amdgcn_exp2f(M[i] - mn);  // 0 while nothing is summed
                    const float wgt = __builtin_amdgcn_exp2f(ms - mn) * ls;
                    Lsum[i] = fmaf(Lsum[i], c, wgt);
                    const uint32_t lo32 = (uint32_t)v[i][x], hi32 = (uint32_t)(v[i][x] >> 32);
                    acc[i][0] = fmaf(acc[i][0], c, wgt * bf16_lo(lo32));
                    acc[i][1] = fmaf(acc[i][1], c, wgt * bf16_hi(lo32));
                    acc[i][2] = fmaf(acc[i][2], c, wgt * bf16_lo(hi32));
                    acc[i][3] = fmaf(acc[i][3], c, wgt * bf16_hi(hi32));
                    M[i] = mn;
                }
        }
#pragma unroll
        for (int i = 0; i < MU; ++i) {
            if (!on[i]) continue;
            const int u = ub + i * kLatThreads;
            const int un = (u >> 6) & 31, ug = (u >> 4) & 3;
            const int hh = HPW * hgi + hl[i];
            const float il = Lsum[i] > 0.f ? 1.f / Lsum[i] : 0.f;
            // agent scope: a failure fill by the group's last split to leave lands after it
            st_agent_u64(a.out + ((int64_t)row * a.heads_q + hh) * kLatV + 16 * un + 4 * ug,
                         (uint64_t)pack_bf16x2(acc[i][0] * il, acc[i][1] * il) |
                             ((uint64_t)pack_bf16x2(acc[i][2] * il, acc[i][3] * il) << 32));
        }
    }
}

// Per tile-phase count T: T = 1 runs 8 waves x 16 heads (128 heads) on every tile; T = 2 runs 4
// head groups x 2 phases (64 heads), the phases taking alternate tiles.
template <int T>
struct LatCfg {
    static constexpr int kRing = 4;                // staged tiles
    static constexpr int kAhead = T == 1 ? 3 : 1;  // steps in flight while one is computed
    // T = 2 keeps a table of logit biases (0 or -inf per selected row); T = 1 derives them from
    // the slot table, whose LDS then holds a fourth tile
    static constexpr bool kBiasTable = T == 2;
    static constexpr int kCPW = T == 1 ? 5 : 9;    // 1 KiB copies per wave per step
    static constexpr int kHPW = 128 / T;           // query heads per workgroup
    static constexpr int kHW = 8 / T;              // groups of 16 heads per workgroup
    static constexpr int kMaxRows = T == 1 ? 2048 : 1024;  // selected rows per split
};

template <int T>
__global__ __launch_bounds__(kLatThreads, 1) void k_attn_latent(AttnArgs a) {
    using C = LatCfg<T>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // dynamic LDS: ring [kRing][36864] | slots [split_len] int32 | (T = 2) logit bias [split_len] fp32
    uint8_t *ring = lds;
    int32_t *s_slot = reinterpret_cast<int32_t *>(lds + C::kRing * kLatTileB);
    float *s_bias = reinterpret_cast<float *>(s_slot + a.split_len);
    __shared__ int s_leave;

    const int tid = threadIdx.x, l = lane_id(), g = l >> 4, L = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hsub = w % C::kHW, tp = w / C::kHW;  // head group of 16, tile phase
    int row, hgi, split;
    lat_unit_of(blockIdx.x, a, row, hgi, split);
    if (row >= a.rows) return;  // padding of the XCD-aligned grid: no barrier counts on it
    int seq, qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int32_t *pt = a.page_table + (int64_t)seq * a.pages_per_seq;
    const int j0 = split * a.split_len;
    const int j1 = min(a.k, j0 + a.split_len);
    const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;
    const int nsteps = (ntiles + T - 1) / T;
    const int P = 1 << a.lp;

    // ---- query fragments (B operand of S^T = K Q^T): head head0 + L, entries 32 s + 8 g + e.
    //      A lane past the last head reads head 0; its column is never stored. Issued first,
    //      so that their latency overlaps the slot-table loads below.
    const int head0 = C::kHPW * hgi + 16 * hsub;
    const int head = head0 + L;
    const bool live_wave = head0 < a.heads_q;
    const bool live = head < a.heads_q;
    //      With T = 2 the two phases of a head group need the same fragments: phase 0 loads
    //      them and hands them to phase 1 through LDS (below).
    u32x4 qf[kLatKS];
    if (T == 1 || tp == 0) {
        const uint16_t *qr = a.q + ((int64_t)row * a.heads_q + (live ? head : 0)) * kLatQK + 8 * g;
#pragma unroll
        for (int s = 0; s < kLatKS; ++s) qf[s] = ldg16(qr + 32 * s);
    }
    // ---- slot and bias of every selected row of this split
    for (int j = tid; j < ntiles * kTile; j += kLatThreads) {
        int32_t slot = -1;
        if (j0 + j < j1) {
            if (a.slots) {
                slot = a.slots[(int64_t)row * a.k + j0 + j];
            } else {
                const int e = a.idx[(int64_t)row * a.k + j0 + j];
                if (e >= 0) slot = pt[e >> a.lp] * P + (e & (P - 1));
            }
        }
        s_slot[j] = slot;
        if constexpr (C::kBiasTable) s_bias[j] = slot < 0 ? -__builtin_inff() : 0.f;
    }
    // every load above completes here (the query fragments included): inside the tile loop the
    // only vector-memory operations in flight are this wave's tile copies, which the waits
    // below count exactly
    __builtin_amdgcn_s_waitcnt(0);
    // T = 2: the query fragments through the ring's slots 2 and 3 ([head group][k-step][lane],
    // 73,728 bytes = two tiles), which the copies of step 1 overwrite only after the loop's first
    // barrier, when every wave has read them
    u32x4 *qx = reinterpret_cast<u32x4 *>(lds + 2 * kLatTileB) + (hsub * kLatKS) * 64 + l;
    if (T == 2 && tp == 0 && live_wave)
#pragma unroll
        for (int s = 0; s < kLatKS; ++s) qx[64 * s] = qf[s];
    __syncthreads();  // the slot table (and the handed-over query fragments) are complete
    if (T == 2 && tp == 1 && live_wave)
#pragma unroll
        for (int s = 0; s < kLatKS; ++s) qf[s] = qx[64 * s];
    // ---- staged tile layout: 16-byte chunk c of row r lives at byte
    //      4096 (c / 8) + 128 r + 16 ((c % 8) ^ swz(r)), i.e. nine column groups of 128 bytes per
    //      row, each group holding the 32 rows. Copy block b (1 KiB) fills group b / 4, rows
    //      8 (b % 4) .. + 7: lane j takes row 8 (b % 4) + j / 8 and position j % 8.
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    // copies of step st (tiles T st .. T st + T - 1, the last tile repeated past the end) into
    // their ring slots. T = 1: 36 blocks per tile over 8 waves, waves 4..7 repeating blocks
    // 32..35 in their fifth copy (the same bytes written twice); T = 2: 72 blocks, 9 per wave.
    auto issue = [&](int st) {
        // recomputed from an opaque lane id: held across the loop these would take registers
        const int lc = (int)opaque((uint32_t)l);
#pragma unroll
        for (int k = 0; k < C::kCPW; ++k) {
            int blk, tin;
            if constexpr (T == 1) {
                blk = k < 4 ? w + 8 * k : 32 + (w & 3);
                tin = 0;
            } else {
                const int q = w + 8 * k;
                tin = q / 36;
                blk = q - 36 * tin;
            }
            const int t = T * st + tin;
            const int tt = min(t, ntiles - 1);
            const uint32_t base = ring_lds + (uint32_t)(t % C::kRing) * kLatTileB;
            const int r = 8 * (blk & 3) + (lc >> 3);
            const int c = 8 * (blk >> 2) + ((lc & 7) ^ swz(r));
            const int32_t slot = s_slot[tt * kTile + r];
            const uint8_t *src = (slot < 0 ? a.zero_row : a.kc + (int64_t)slot * kLatRowB) + 16 * c;
            copy16_to_lds(src, __builtin_amdgcn_readfirstlane(base + 1024u * (uint32_t)blk));
        }
    };

    f32x4 o[kLatDT];
#pragma unroll
    for (int n = 0; n < kLatDT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;

    if (nsteps > 0)
#pragma unroll
        for (int st = 0; st < C::kAhead; ++st) issue(st);
    for (int st = 0; st < nsteps; ++st) {
        if constexpr (T == 1) {
            // step st has landed once at most the copies of steps st + 1 .. st + kAhead - 1 are
            // outstanding
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((C::kAhead - 1) * C::kCPW));
            lds_barrier();            // every wave's copies of step st landed; st - 1 fully read
            issue(st + C::kAhead);    // into the slots step st - 1 occupied
        } else {
            // one step ahead only: its copies go out before this step's wait, so that the pipe
            // never drains
            lds_barrier();            // step st - 1 fully read: its slots are free
            issue(st + C::kAhead);    // into the slots step st - 1 occupied
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kAhead * C::kCPW));
            lds_barrier();            // every wave's copies of step st landed
        }
        const int t = T * st + tp;
        if (!live_wave || t >= ntiles) continue;
        const uint32_t kb = ring_lds + (uint32_t)(t % C::kRing) * kLatTileB;
        // ---- S^T over the 576-wide contraction: two 16-row M tiles. Key fragment of k-step s,
        //      M tile mt: row 16 mt + L, chunk 4 s + g = 8 (s / 2) + (4 (s % 2) + g): column group
        //      s / 2 is an immediate offset, the swizzle touches the second part only. The bases
        //      are recomputed per tile from an opaque lane id (held across the loop they would
        //      take registers). Reads run kKA steps ahead of their MFMA.
        constexpr int kKA = 4;
        f32x4 sa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        uint32_t kbase[2][2];
        {
            const uint32_t lo = opaque((uint32_t)l), Lo = lo & 15u, go = lo >> 4;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    const int r = 16 * mt + (int)Lo;
                    kbase[mt][sp] = kb + (uint32_t)(128 * r + 16 * ((4 * sp + (int)go) ^ swz(r)));
                }
        }
        auto kread = [&](int i) {  // step i = 2 s + mt
            const int s = i >> 1, mt = i & 1;
            return *reinterpret_cast<const SA_LDS u32x4 *>(kbase[mt][s & 1] + 4096u * (uint32_t)(s >> 1));
        };
        u32x4 kf[kKA];
#pragma unroll
        for (int i = 0; i < kKA; ++i) kf[i] = kread(i);
#pragma unroll
        for (int i = 0; i < 2 * kLatKS; ++i) {
            const u32x4 cur = kf[i % kKA];
            if (i + kKA < 2 * kLatKS) kf[i % kKA] = kread(i + kKA);
            sa[i & 1] = mfma16x16x32(cur, qf[i >> 1], sa[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- logits in the log2 domain: rows 16 mt + 4 g + i of head L
        f32x4 b0, b1;
        if constexpr (C::kBiasTable) {
            const float *bia = s_bias + t * kTile + 4 * g;
            b0 = *reinterpret_cast<const f32x4 *>(bia);
            b1 = *reinterpret_cast<const f32x4 *>(bia + 16);
        } else {
            const int32_t *sli = s_slot + t * kTile + 4 * g;
            const u32x4 q0 = *reinterpret_cast<const u32x4 *>(sli);
            const u32x4 q1 = *reinterpret_cast<const u32x4 *>(sli + 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b0[i] = (int32_t)q0[i] < 0 ? -__builtin_inff() : 0.f;
                b1[i] = (int32_t)q1[i] < 0 ? -__builtin_inff() : 0.f;
            }
        }
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = fmaf(sa[0][i], a.scale_log2, b0[i]);
            x[4 + i] = fmaf(sa[1][i], a.scale_log2, b1[i]);
        }
        float m_tile = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        m_tile = fmaxf(m_tile, __shfl_xor(m_tile, 16, 64));
        m_tile = max_xor32(m_tile);
        const bool grow = m_tile > m_run + kRescale;
        if (__any(grow)) {
            const float m_new = grow ? m_tile : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < kLatDT; ++n) o[n] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
            l_run += p[e];
        }
        // P^T B operand: k = 8 g + e <-> the lane's own rows, in the order of the V reads below:
        // e = 0..3 rows 4g, 4g+1, 16+4g, 16+4g+1; e = 4..7 the same plus 2
        const u32x4 pb = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[2], p[3]), pack_bf16x2(p[6], p[7])};
        // ---- O^T += V^T P^T. Transposing reads: input lane J of group g loads entries
        //      [4 (J % 4), +4) of row R(J / 4), R(q) = 4 g + (q & 1) + 16 (q >> 1) (+ 2 for the
        //      second read); output lane L then holds entry L of rows R(0) .. R(3). Chunk
        //      2 n + (L % 4) / 2 = 8 (n / 4) + (2 (n % 4) + (L % 4) / 2): column group n / 4 is an
        //      immediate offset, four bases per read row. Reads run kVA tiles ahead of their MFMA.
        constexpr int kVA = 3;
        uint32_t vbase[2][4];
        {
            const uint32_t l2 = opaque((uint32_t)l), L2 = l2 & 15u, g2 = l2 >> 4;
            const int q = (int)(L2 >> 2);
            const int vr1 = 4 * (int)g2 + (q & 1) + 16 * (q >> 1);
#pragma unroll
            for (int rd = 0; rd < 2; ++rd)
#pragma unroll
                for (int nq = 0; nq < 4; ++nq) {
                    const int vr = vr1 + 2 * rd;
                    vbase[rd][nq] = kb + (uint32_t)(128 * vr +
                                                    16 * ((2 * nq + (int)((L2 & 3u) >> 1)) ^ swz(vr)) +
                                                    8 * (int)(L2 & 1u));
                }
        }
        auto vread = [&](int n) {
            const uint32_t off = 4096u * (uint32_t)(n >> 2);
            const u32x2 w0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                           (SA_LDS i16x4 *)(vbase[0][n & 3] + off)));
            const u32x2 w1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                           (SA_LDS i16x4 *)(vbase[1][n & 3] + off)));
            return u32x4{w0[0], w0[1], w1[0], w1[1]};
        };
        u32x4 vf[kVA];
#pragma unroll
        for (int n = 0; n < kVA; ++n) vf[n] = vread(n);
#pragma unroll
        for (int n = 0; n < kLatDT; ++n) {
            const u32x4 cur = vf[n % kVA];
            if (n + kVA < kLatDT) vf[n % kVA] = vread(n + kVA);
            o[n] = mfma16x16x32(cur, pb, o[n]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the copies issued past the last step land before the ring is reused or released
    __builtin_amdgcn_s_waitcnt(0);

    // ---- T = 2: phase 1 hands its (max, sum, output) to phase 0 of the same head group through
    //      the ring (free now), which combines the two with the usual rescaling. Both phases hold
    //      the same entries per lane, so the combination is lane by lane.
    if constexpr (T == 2) {
        float *xo = reinterpret_cast<float *>(ring);      // [4 groups][32 n][64 lanes][4]
        float *xm = xo + C::kHW * kLatDT * 64 * 4;        // [4 groups][64 lanes] max, then sum
        __syncthreads();  // every wave has finished reading the ring
        if (tp == 1 && live_wave) {
#pragma unroll
            for (int n = 0; n < kLatDT; ++n)
                *reinterpret_cast<f32x4 *>(xo + ((hsub * kLatDT + n) * 64 + l) * 4) = o[n];
            xm[hsub * 64 + l] = m_run;
            xm[C::kHW * 64 + hsub * 64 + l] = l_run;
        }
        __syncthreads();
        if (tp == 0 && live_wave) {
            const float m1 = xm[hsub * 64 + l], l1 = xm[C::kHW * 64 + hsub * 64 + l];
            const float M = fmaxf(m_run, m1);
            const bool none = M == -__builtin_inff();
            const float a0 = none || m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
            const float a1 = none || m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
            l_run = l_run * a0 + l1 * a1;
#pragma unroll
            for (int n = 0; n < kLatDT; ++n) {
                const f32x4 v1 = *reinterpret_cast<const f32x4 *>(xo + ((hsub * kLatDT + n) * 64 + l) * 4);
                o[n] = o[n] * a0 + v1 * a1;
            }
            m_run = M;
        }
    }
    const bool owner = tp == 0;  // the waves that hold the workgroup's result

    // ---- epilogue: lane (g, L) holds entries 16 n + 4 g + i of head L
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot = sum_xor32(l_tot);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (!a.merge_inside) {
        if (owner && live) {
            uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * kLatV;
#pragma unroll
            for (int n = 0; n < kLatDT; ++n)
                *reinterpret_cast<u32x2 *>(orow + 16 * n + 4 * g) =
                    u32x2{pack_bf16x2(o[n][0] * inv, o[n][1] * inv),
                          pack_bf16x2(o[n][2] * inv, o[n][3] * inv)};
        }
        return;
    }
    // ---- split partials (agent scope, see st_agent_u64), then the barrier of the (row, head
    //      group). A split's partial output is a block of 8-byte units (four bf16), unit
    //      u = ((hsub * 32 + n) * 4 + g) * 16 + L holding entries 16 n + 4 g .. + 3 of head
    //      head0 + L: each store instruction of a wave writes 512 contiguous bytes. Blocks of
    //      one head group hold blk_heads heads (the head count rounded up to 16 when there is
    //      one group).
    const int blk_heads = a.hgroups == 1 ? 16 * ((a.heads_q + 15) / 16) : C::kHPW;
    const int64_t blk_elems = (int64_t)blk_heads * kLatV;
    const int64_t grp = (int64_t)row * a.hgroups + hgi;  // (row, head group)
    if (owner && live_wave) {
        uint16_t *pblk = a.part_o + (grp * a.splits + split) * blk_elems;
#pragma unroll
        for (int n = 0; n < kLatDT; ++n) {
            const uint64_t v = (uint64_t)pack_bf16x2(o[n][0] * inv, o[n][1] * inv) |
                               ((uint64_t)pack_bf16x2(o[n][2] * inv, o[n][3] * inv) << 32);
            st_agent_u64(pblk + 4 * (((hsub * kLatDT + n) * 4 + g) * 16 + L), v);
        }
        if (g == 0 && live)
            st_agent_u64(a.part_ml + 2 * ((grp * a.splits + split) * C::kHPW + 16 * hsub + L),
                         (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_tot) << 32));
    }
    uint32_t *rs = a.row_sync + grp * kRowSyncWords;
    uint32_t nbar = 0;
    const bool ok = group_barrier(&rs[0], (uint32_t)a.splits, a.err, nbar, a.spin_limit);
    // ---- merge: split s combines the units [s U / S, (s + 1) U / S) of every split's block
    //      (U = units per block). Consecutive threads take consecutive units; a thread issues
    //      the loads of MU units (kLatThreads apart) for MS splits before it combines any: with
    //      few splits 4 units x 4 splits, with many 1 unit x 16 splits, so that one memory round
    //      trip usually covers everything a thread merges.
    const int units = blk_heads * kLatV / 4;
    const int u0 = (int)((int64_t)units * split / a.splits);
    const int u1 = (int)((int64_t)units * (split + 1) / a.splits);
    if (ok) {
        if (a.splits <= 4)
            lat_merge_units<C::kHPW, 4, 4>(a, row, hgi, grp, blk_elems, u0, u1);
        else
            lat_merge_units<C::kHPW, 1, 16>(a, row, hgi, grp, blk_elems, u0, u1);
    } else if (tid == 0) {
        __hip_atomic_fetch_or(&rs[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // ---- leave: the last split to leave (all others have written everything) resets the
    //      record; if any split's wait expired, it also zeroes the group's whole output, so a
    //      failed call leaves a defined result (zeros, with bit 0 of the error word set)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&rs[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_leave = prev == (uint32_t)a.splits - 1 ? 1 + (int)ld_agent(&rs[2]) : 0;
    }
    __syncthreads();
    if (s_leave == 2) {  // last to leave, after a failure
        const int h0 = C::kHPW * hgi, h1 = min(a.heads_q, h0 + C::kHPW);
        uint16_t *orow = a.out + ((int64_t)row * a.heads_q + h0) * kLatV;
        for (int i = tid; i < (h1 - h0) * kLatV / 4; i += kLatThreads) st_agent_u64(orow + 4 * i, 0ull);
    }
    if (s_leave >= 1 && tid == 0) {
        st_agent(&rs[0], 0u);
        st_agent(&rs[1], 0u);
        st_agent(&rs[2], 0u);
    }
}

size_t attn_latent_lds(int tphases, int split_len) {
    const int ring = tphases == 1 ? LatCfg<1>::kRing : LatCfg<2>::kRing;
    const bool bias = tphases == 1 ? LatCfg<1>::kBiasTable : LatCfg<2>::kBiasTable;
    return (size_t)ring * kLatTileB + (size_t)split_len * (bias ? 8 : 4);
}

int attn_latent_max_rows(int tphases) {
    return tphases == 1 ? LatCfg<1>::kMaxRows : LatCfg<2>::kMaxRows;
}

template <int T>
static hipError_t launch_latent_t(const AttnArgs &a, hipStream_t st) {
    const size_t lds = attn_latent_lds(T, a.split_len);
    static std::atomic<int> granted{-1};
    hipError_t e = hipSuccess;
    if ((int)lds > granted.load(std::memory_order_relaxed)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_attn_latent<T>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        granted.store((int)lds, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL(k_attn_latent<T>,
                       dim3((unsigned)lat_grid(a.rows, a.hgroups * a.splits, a.xcd_align)),
                       dim3(kLatThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_attn_latent(const AttnArgs &a, int tphases, hipStream_t st) {
    if (tphases == 1) return launch_latent_t<1>(a, st);
    if (tphases == 2) return launch_latent_t<2>(a, st);
    return hipErrorInvalidValue;
}

int lat_grid_host(int rows, int units, int xcd_align) { return lat_grid(rows, units, xcd_align); }

int attn_latent_occupancy(int tphases, int split_len) {
    int occ = 0;
    const void *kern = tphases == 1 ? reinterpret_cast<const void *>(&k_attn_latent<1>)
                                    : reinterpret_cast<const void *>(&k_attn_latent<2>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kLatThreads,
                                                     attn_latent_lds(tphases, split_len)) != hipSuccess)
        return -1;
    return occ;
}

template <int DQK, int DV, bool SEPV, bool FP8, bool T128 = false>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
    constexpr int NSC = T128 ? (DQK + 127) / 128 : (FP8 ? 1 : 0);  // scales per staged row
    const size_t lds = (size_t)4 * 2 * 2 * 64 * 16 + (size_t)a.split_len * (8 + 4 * NSC);
    auto kern = k_sparse_attn_pairs<DQK, DV, SEPV, FP8, T128>;
    // raise the kernel's dynamic-LDS limit only when a launch needs more than already granted
    static std::atomic<int> granted{-1};
    hipError_t e = hipSuccess;
    if ((int)lds > granted.load(std::memory_order_relaxed)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        granted.store((int)lds, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.rows * a.splits * a.hgroups)), dim3(512), lds, st,
                       a);
    e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(k_attn_merge<DV>, dim3((unsigned)a.rows, (unsigned)((a.heads_q + 3) / 4)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs &a, int dqk, int dv, bool sep_v, int kv_fmt,
                              hipStream_t st) {
    const bool fp8 = kv_fmt != 0;
    if (dqk == 576 && dv == 512 && !sep_v) {
        if (kv_fmt == 3) return launch_attn_t<576, 512, false, true, true>(a, st);
        return fp8 ? launch_attn_t<576, 512, false, true>(a, st)
                   : launch_attn_t<576, 512, false, false>(a, st);
    }
    if (dqk == 128 && dv == 128 && !fp8)
        return sep_v ? launch_attn_t<128, 128, true, false>(a, st)
                     : launch_attn_t<128, 128, false, false>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace sa
