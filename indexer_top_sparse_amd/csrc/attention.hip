// Sparse attention over the gathered rows of the selected positions, gfx950.
//
// "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei
// Ascend CANN Architecture" §1 and §2.1 (the attention reads the KV precisely according to the
// selected indices); "Engineering Path for Day-0 Adaptation of Trillion-Scale Sparse Models on
// Domestic AI Accelerators" §3.1-§3.2 (non-contiguous access by index; block number + offset).
//
// One workgroup = one query row x one split of its index list, 32 query heads per wave. All
// heads share one KV row (MQA / MLA latent rows), so each gathered row is staged once in LDS
// and used by every wave:
//   S^T[tok][head] = K[tok][:] . Q[head][:]          (32x32x16 bf16 MFMA, K from LDS)
//   online softmax per head (lazy rescaling; a lane holds 16 tokens of one head)
//   O^T[d][head]  += V^T[d][tok] . P^T[tok][head]    (V^T fragments by transposing LDS reads)
// Splits write unnormalised partials that k_attn_merge combines.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTile = 32;          // gathered rows per iteration
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
    static constexpr int CPR_K = ROWB_K / 16;            // 16-byte LDS chunks per row
    static constexpr int CPR_V = SEPV ? ROWB_V / 16 : 0;
    static constexpr int KBUF = kTile * ROWB_K;
    static constexpr int BUF = KBUF + (SEPV ? kTile * ROWB_V : 0);
    static constexpr int NCHUNK = kTile * (CPR_K + CPR_V);  // LDS chunks per tile
    // a direct-to-LDS instruction always fills 64 chunks: tiles must be whole instructions
    static_assert(NCHUNK % 64 == 0, "staged tile must be a multiple of 64 chunks");
};

// One workgroup = NP wave pairs of one head group; pair p owns query heads
// [32 (NP hg + p), +32). The two waves of a
// pair split the QK^T contraction over d (each adds half of the k-steps; the partial scores
// are exchanged through LDS) and split the PV output over d_v, so each wave holds half of the
// query fragments and half of the output accumulator.
template <int NP, int DQK, int DV, bool SEPV, bool FP8>
__global__ __launch_bounds__(128 * NP) void k_sparse_attn(AttnArgs a) {
    using S = AttnShape<DQK, DV, SEPV, FP8>;
    constexpr int NT = 128 * NP;
    constexpr int KS = DQK / 16 / 2;   // k-steps per wave
    constexpr int ND = DV / 32 / 2;    // 32-wide d_v tiles per wave
    constexpr int NWV = 2 * NP;

    // Staging buffers as separate objects: the loop rotates through them at compile time, so
    // the compiler can tell that the reads of one never alias the global->LDS copies into the
    // others and keeps those copies in flight across the reads. bf16 rows use a ring of three
    // (two tiles in flight); E4M3 rows, staged through registers, use two.
    __shared__ __attribute__((aligned(16))) uint8_t stage_a[S::BUF];
    __shared__ __attribute__((aligned(16))) uint8_t stage_b[S::BUF];
    __shared__ __attribute__((aligned(16))) uint8_t stage_c[FP8 ? 16 : S::BUF];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // dynamic lds: [NWV][32][32] fp32 partial scores | [split_len] int32 slots |
    //              [split_len] fp32 row flags (scale or 1; < 0 empty)
    float *s_part = reinterpret_cast<float *>(lds);
    int32_t *s_slot = reinterpret_cast<int32_t *>(lds + NWV * 4096);
    float *s_sig = reinterpret_cast<float *>(s_slot + a.split_len);

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int h = l >> 5, lm = l & 31;
    const int pair = w >> 1, half = w & 1;
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
        s_sig[j] = slot < 0 ? -1.f : (FP8 ? a.kv_scale[slot] : 1.f);
    }

    // query fragments (B operand of S^T = K Q^T): head 32 (NP hg + pair) + l%32,
    // d = 16s + 8h + e for this wave's k-steps s in [half*KS, half*KS + KS)
    const int head = 32 * (NP * hg + pair) + lm;
    u32x4 qf[KS];
    {
        const uint16_t *qr = a.q + ((int64_t)row * a.heads_q + head) * DQK + 8 * h;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = head < a.heads_q ? ldg16(qr + 16 * (half * KS + s)) : u32x4{0u, 0u, 0u, 0u};
    }

    // Gather of tile t into LDS buffer `buf`. bf16 rows go global -> LDS directly (lane i of an
    // instruction fills LDS chunk base + i; the swizzle is applied on the global side); empty
    // rows read a zero row. E4M3 rows go through registers and are widened to bf16.
    constexpr int FP8_CH = kTile * (DQK / 16);  // 16-byte global chunks of a fp8 tile
    constexpr int FP8_PER = (FP8_CH + NT - 1) / NT;
    u32x4 stg[FP8 ? FP8_PER : 1];
    auto gather = [&](int t, uint8_t *base) {
        const int32_t *slots = s_slot + t * kTile;
        if (!FP8) {
            for (int ins = w; ins * 64 < S::NCHUNK; ins += NWV) {
                const int ch = ins * 64 + l;
                const bool isv = SEPV && ch >= kTile * S::CPR_K;
                const int cc = isv ? ch - kTile * S::CPR_K : ch;
                const int cpr = isv ? S::CPR_V : S::CPR_K;
                const int r = cc / cpr, c = cc % cpr;
                const int32_t slot = slots[r];
                const uint8_t *src = a.zero_row;
                if (slot >= 0)
                    src = (isv ? a.vc + (int64_t)slot * S::VROW_G
                               : a.kc + (int64_t)slot * S::KROW_G) +
                          16 * (c ^ swz(r));
                __builtin_amdgcn_global_load_lds(src, (SA_LDS void *)(base + ins * 1024), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < FP8_PER; ++i) {
                const int c = tid + i * NT;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (c < FP8_CH) {
                    const int r = c / (DQK / 16), col = c % (DQK / 16);
                    const int32_t slot = slots[r];
                    if (slot >= 0) v = ldg16(a.kc + (int64_t)slot * S::KROW_G + 16 * col);
                }
                stg[i] = v;
            }
        }
    };
    auto stage_fp8 = [&](uint8_t *kb) {
        if (FP8) {
#pragma unroll
            for (int i = 0; i < FP8_PER; ++i) {
                const int c = tid + i * NT;
                if (c < FP8_CH) {
                    const int r = c / (DQK / 16), col = c % (DQK / 16);
                    const u32x2 q0 = e4m3x4_to_bf16(stg[i][0]), q1 = e4m3x4_to_bf16(stg[i][1]);
                    const u32x2 q2 = e4m3x4_to_bf16(stg[i][2]), q3 = e4m3x4_to_bf16(stg[i][3]);
                    uint8_t *rowp = kb + r * S::ROWB_K;
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col) ^ swz(r))) =
                        u32x4{q0[0], q0[1], q1[0], q1[1]};
                    *reinterpret_cast<u32x4 *>(rowp + 16 * ((2 * col + 1) ^ swz(r))) =
                        u32x4{q2[0], q2[1], q3[0], q3[1]};
                }
            }
        }
    };

    f32x16 o[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;

    __syncthreads();  // slot table ready
    // this wave's global->LDS copy instructions per tile (the last tile's loads that a wave
    // may leave in flight at the end-of-tile wait)
    constexpr int NI_MIN = (S::NCHUNK / 64) / NWV;
    if (ntiles > 0) {
        gather(0, stage_a);
        if (!FP8 && ntiles > 1) gather(1, stage_b);
        stage_fp8(stage_a);
        if (!FP8) {
            // tile 0 landed (tile 1's copies, issued last, may still be in flight)
            if (ntiles > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI_MIN));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        full_barrier_lds_only_after_wait();
    }
    const int g = l >> 4, jj = l & 15;
    auto tile = [&](int t, const uint8_t *kb, uint8_t *next) {
        // bf16: copy tile t+2 into the buffer of tile t-1 (free since the last barrier);
        // E4M3: load tile t+1 into registers, widened into `next` at the end
        if (FP8) {
            if (t + 1 < ntiles) gather(t + 1, next);
        } else {
            if (t + 2 < ntiles) gather(t + 2, next);
        }

        const uint8_t *vb = SEPV ? kb + S::KBUF : kb;
        constexpr int VROWB = SEPV ? S::ROWB_V : S::ROWB_K;
        // ---- partial S^T = K Q^T over this wave's half of d: two independent accumulation
        //      chains (even / odd k-steps), fragment reads running ahead
        f32x16 sacc, sacc2;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = sacc2[r] = 0.f;
        const uint8_t *krow = kb + lm * S::ROWB_K;
        const int sw = swz(lm);
        auto kfrag = [&](int s) {
            const int c = 2 * (half * KS + s) + h;
            return *reinterpret_cast<const u32x4 *>(krow + 16 * (c ^ sw));
        };
        u32x4 ka = kfrag(0), kb2 = kfrag(1);
#pragma unroll
        for (int s = 0; s < KS; s += 2) {
            const u32x4 a0 = ka, a1 = kb2;
            if (s + 2 < KS) ka = kfrag(s + 2);
            if (s + 3 < KS) kb2 = kfrag(s + 3);
            sacc = mfma32x32x16(a0, qf[s], sacc);
            if (s + 1 < KS) sacc2 = mfma32x32x16(a1, qf[s + 1], sacc2);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] += sacc2[r];
        // exchange partial scores with the other wave of the pair
        float *mine = s_part + (w * 32 + lm) * 32 + 16 * h;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4 *>(mine + 4 * q4) =
                f32x4{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
        lds_barrier();
        // both waves add in the same order (a + b == b + a), so their softmax states agree;
        // logits in the log2 domain, -inf for empty rows
        const float *theirs = s_part + ((w ^ 1) * 32 + lm) * 32 + 16 * h;
        const float *sig = s_sig + t * kTile;
        float m_tile = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 ov = *reinterpret_cast<const f32x4 *>(theirs + 4 * j);
            const f32x4 sv = *reinterpret_cast<const f32x4 *>(sig + 8 * j + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                const float v = (sacc[r] + ov[i]) * a.scale_log2 * (FP8 ? sv[i] : 1.f);
                sacc[r] = sv[i] < 0.f ? -__builtin_inff() : v;
                m_tile = fmaxf(m_tile, sacc[r]);
            }
        }
        m_tile = fmaxf(m_tile, __shfl_xor(m_tile, 32, 64));
        const bool grow = m_tile > m_run + kRescale;
        if (__any(grow)) {
            const float m_new = grow ? m_tile : m_run;
            // alpha = 0 when m_run = -inf (nothing accumulated yet)
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < ND; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[n][r] *= alpha;
            m_run = m_new;
        }
        // exp2(-inf - m) = 0 for empty rows; m_run is finite once any row was seen, and while
        // it is -inf every logit is -inf too, which the select below maps to 0
        const bool none = m_run == -__builtin_inff();
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
                    const float p = none ? 0.f : __builtin_amdgcn_exp2f(sacc[r] - m_run);
                    l_run += p;
                    pp[e1] = FP8 ? p * fmaxf(sig[8 * (r >> 2) + 4 * h + (r & 3)], 0.f) : p;
                }
                pk[e2] = pack_bf16x2(pp[0], pp[1]);
            }
            pb[u] = u32x4{pk[0], pk[1], pk[2], pk[3]};
        }
        // ---- O^T += V^T P^T over this wave's half of d_v: two 16-token k-steps
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ra = 16 * u + 4 * (g >> 1) + (jj >> 2), rb = ra + 8;
            const uint8_t *va = vb + ra * VROWB, *vbp = vb + rb * VROWB;
            const int swa = swz(ra), swb = swz(rb);
            const int byte_in = 8 * (jj & 1);
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                const int c = 4 * (half * ND + n) + 2 * (g & 1) + ((jj & 3) >> 1);
                const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SA_LDS i16x4 *)(va + 16 * (c ^ swa) + byte_in));
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SA_LDS i16x4 *)(vbp + 16 * (c ^ swb) + byte_in));
                const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
                const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
                o[n] = mfma32x32x16(u32x4{w0[0], w0[1], w1[0], w1[1]}, pb[u], o[n]);
            }
        }
        if (FP8) {
            if (t + 1 < ntiles) stage_fp8(next);
            full_barrier();  // tile t+1 staged; everyone is done with this buffer
        } else {
            // tile t+1 has landed once at most this wave's copies of tile t+2 are in flight
            if (t + 2 < ntiles) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI_MIN));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            full_barrier_lds_only_after_wait();
        }
    };
    if (FP8) {
        for (int t = 0; t < ntiles; t += 2) {
            tile(t, stage_a, stage_b);
            if (t + 1 < ntiles) tile(t + 1, stage_b, stage_a);
        }
    } else {
        // tile t reads buffer t % 3 and copies tile t+2 into buffer (t+2) % 3
        for (int t = 0; t < ntiles; t += 3) {
            tile(t, stage_a, stage_c);
            if (t + 1 < ntiles) tile(t + 1, stage_b, stage_a);
            if (t + 2 < ntiles) tile(t + 2, stage_c, stage_b);
        }
    }

    // ---- epilogue: this wave owns d_v tiles [half*ND, half*ND + ND) of head `head`
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (head >= a.heads_q) return;
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * DV;
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * (half * ND + n) + 8 * j + 4 * h;
                u32x2 v = {pack_bf16x2(o[n][4 * j] * inv, o[n][4 * j + 1] * inv),
                           pack_bf16x2(o[n][4 * j + 2] * inv, o[n][4 * j + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + d) = v;
            }
    } else {
        const int64_t ph = ((int64_t)row * a.splits + split) * a.heads_q + head;
        float *orow = a.part_o + ph * DV;
#pragma unroll
        for (int n = 0; n < ND; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 32 * (half * ND + n) + 8 * j + 4 * h;
                *reinterpret_cast<f32x4 *>(orow + d) =
                    f32x4{o[n][4 * j], o[n][4 * j + 1], o[n][4 * j + 2], o[n][4 * j + 3]};
            }
        if (h == 0 && half == 0) {
            a.part_ml[2 * ph] = m_run;
            a.part_ml[2 * ph + 1] = l_tot;
        }
    }
}

// Combine split partials: o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Grid: rows x ceil(heads/4); 256 threads = 4 heads x 64 threads x (DV/64) entries.
template <int DV>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
    constexpr int PER = DV / 64;
    const int row = blockIdx.x;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (head >= a.heads_q) return;
    const int d0 = (threadIdx.x & 63) * PER;
    float M = -__builtin_inff();
    for (int s = 0; s < a.splits; ++s)
        M = fmaxf(M, a.part_ml[2 * (((int64_t)row * a.splits + s) * a.heads_q + head)]);
    float L = 0.f, acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s = 0; s < a.splits; ++s) {
        const int64_t ph = ((int64_t)row * a.splits + s) * a.heads_q + head;
        const float m = a.part_ml[2 * ph], lv = a.part_ml[2 * ph + 1];
        if (lv == 0.f) continue;
        const float wgt = exp2f(m - M);
        L += wgt * lv;
        const float *po = a.part_o + ph * DV + d0;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += wgt * po[e];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t *orow = a.out + ((int64_t)row * a.heads_q + head) * DV + d0;
#pragma unroll
    for (int e = 0; e < PER; e += 2)
        *reinterpret_cast<uint32_t *>(orow + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
}

template <int NP, int DQK, int DV, bool SEPV, bool FP8>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
    const size_t lds = (size_t)2 * NP * 4096 + (size_t)a.split_len * 8;
    auto kern = k_sparse_attn<NP, DQK, DV, SEPV, FP8>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.rows * a.splits * a.hgroups)), dim3(128 * NP), lds,
                       st, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(k_attn_merge<DV>, dim3((unsigned)a.rows, (unsigned)((a.heads_q + 3) / 4)),
                       dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs &a, int dqk, int dv, bool sep_v, bool fp8,
                              hipStream_t st) {
    const int np = attn_pairs(a.heads_q);
#define SA_ATTN_NP(DQK, DV, SEPV, FP8)                                         \
    if (np == 1) return launch_attn_t<1, DQK, DV, SEPV, FP8>(a, st);           \
    return launch_attn_t<2, DQK, DV, SEPV, FP8>(a, st);
    if (dqk == 576 && dv == 512 && !sep_v) {
        if (fp8) { SA_ATTN_NP(576, 512, false, true) }
        SA_ATTN_NP(576, 512, false, false)
    }
    if (dqk == 128 && dv == 128 && !fp8) {
        if (sep_v) { SA_ATTN_NP(128, 128, true, false) }
        SA_ATTN_NP(128, 128, false, false)
    }
#undef SA_ATTN_NP
    return hipErrorInvalidValue;
}

}  // namespace sa
