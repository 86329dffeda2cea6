// Indexer prolog on gfx950: the three projections that feed the indexer (query, key, head
// weights) as one grid of 16-column tiles, then the key's LayerNorm.
//
// "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei
// Ascend CANN Architecture" (CANN) §2.2: Q projection with K normalization, and Q quantization
// with the head-weight projection, run as independent work before the indexer. Here the
// independent projections share one launch (their tiles fill the device together instead of
// three streams each holding part of it); Q quantization happens inside the MXFP8 indexer.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kPlThreads = 256;  // 4 waves; each takes a quarter of the contraction

// Tile jobs, in launch order (the long contractions first): key columns, head-weight columns,
// then query columns; 16 output columns each.
struct PlJob {
    int kind;  // 0 key (pre-norm, fp32 scratch), 1 head weights (fp32), 2 query (bf16)
    int n0, N, K;
    const uint16_t *x, *w;
};

__device__ __forceinline__ PlJob pl_job(const PrologArgs &a, int t) {
    const int nk = (a.dim + 15) / 16, nw = (a.heads + 15) / 16;
    if (t < nk) return {0, 16 * t, a.dim, a.d_model, a.x, a.w_k};
    t -= nk;
    if (t < nw) return {1, 16 * t, a.heads, a.d_model, a.x, a.w_w};
    t -= nw;
    return {2, 16 * t, a.heads * a.dim, a.d_q, a.x_q, a.w_q};
}

// y[m][n] = sum_k x[m][k] * W[n][k] for MT 16-row tiles starting at row m0 and the job's 16
// columns. MFMA 16x16x32: A = x (lane l: row l%16, k = 8(l/16)..), B = W^T (lane l: column
// l%16, the same k). Rows and columns past the ends read the last valid row (loads stay
// unconditional) and are not stored.
template <int MT>
__global__ __launch_bounds__(kPlThreads) void k_prolog_gemm(PrologArgs a, int m0) {
    __shared__ f32x4 red[4][MT][64];
    const PlJob j = pl_job(a, blockIdx.x);
    const int l = lane_id(), w = wave_id(), g = l >> 4;
    const int n = min(j.n0 + (l & 15), j.N - 1);
    const int kq = j.K / 4;  // this wave's quarter of the contraction (a multiple of 32)
    const uint16_t *wp = j.w + (size_t)n * j.K + (size_t)w * kq + 8 * g;
    const uint16_t *xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xp[mt] = j.x + (size_t)min(m0 + 16 * mt + (l & 15), a.rows - 1) * j.K + (size_t)w * kq + 8 * g;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // k-steps of 32 in groups of U, two groups in flight: the loads of group s + 1 are issued
    // before group s is multiplied. Every group issues the same loads (a group past the end
    // re-reads the last one), so the wait before each group is exact.
    constexpr int U = 4;
    const int ng = (kq / 32 + U - 1) / U;  // groups
    const int last = kq / 32 - 1;          // last k-step
    u32x4 b[2][U], xf[2][U][MT];
    auto load = [&](int buf, int grp) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ks = 32 * min(grp * U + u, last);
            b[buf][u] = ldg16_stream(wp + ks);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xf[buf][u][mt] = ldg16(xp[mt] + ks);
        }
    };
    auto mul = [&](int buf, int grp) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (grp * U + u <= last)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32(xf[buf][u][mt], b[buf][u], acc[mt]);
    };
    load(0, 0);
    for (int grp = 0; grp < ng; grp += 2) {
        load(1, grp + 1);
        mul(0, grp);
        load(0, grp + 2);
        mul(1, grp + 1);
    }
    // sum the four quarters: wave w adds up M-tiles w, w + 4, ...
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][mt][l] = acc[mt];
    __syncthreads();
    const int col = j.n0 + (l & 15);
    for (int mt = w; mt < MT; mt += 4) {
        f32x4 s = red[0][mt][l];
#pragma unroll
        for (int v = 1; v < 4; ++v) s += red[v][mt][l];
        if (col >= j.N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * mt + 4 * g + i;
            if (m >= a.rows) continue;
            if (j.kind == 0) a.k_pre[(size_t)m * a.dim + col] = s[i];
            else if (j.kind == 1) a.w_out[(size_t)m * a.heads + col] = s[i];
            else a.q_out[(size_t)m * a.heads * a.dim + col] = (uint16_t)(pack_bf16x2(s[i], 0.f) & 0xFFFFu);
        }
    }
}

// LayerNorm of one row of the pre-norm key (fp32): mean, then the mean of squared deviations,
// (y - mean) / sqrt(var + eps) * gamma + beta, rounded to bf16. One wave per row.
__global__ __launch_bounds__(64) void k_prolog_norm(PrologArgs a) {
    const int row = blockIdx.x, l = lane_id();
    const float *y = a.k_pre + (size_t)row * a.dim;
    const int D = a.dim;  // <= 128: two entries per lane
    const float y0 = l < D ? y[l] : 0.f, y1 = l + 64 < D ? y[l + 64] : 0.f;
    float s = y0 + y1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    const float mu = s / (float)D;
    const float d0 = l < D ? y0 - mu : 0.f, d1 = l + 64 < D ? y1 - mu : 0.f;
    float v = d0 * d0 + d1 * d1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const float inv = 1.f / sqrtf(v / (float)D + a.eps);
    uint16_t *out = a.k_out + (size_t)row * D;
    if (l < D) out[l] = (uint16_t)(pack_bf16x2(d0 * inv * a.gamma[l] + a.beta[l], 0.f) & 0xFFFFu);
    if (l + 64 < D)
        out[l + 64] = (uint16_t)(pack_bf16x2(d1 * inv * a.gamma[l + 64] + a.beta[l + 64], 0.f) & 0xFFFFu);
}

hipError_t launch_prolog(const PrologArgs &a, hipStream_t st) {
    const int tiles = (a.dim + 15) / 16 + (a.heads + 15) / 16 + (a.heads * a.dim + 15) / 16;
    for (int m0 = 0; m0 < a.rows; m0 += 64) {
        const int mt = min(4, (a.rows - m0 + 15) / 16);
        auto kern = mt == 1 ? k_prolog_gemm<1> : mt == 2 ? k_prolog_gemm<2>
                  : mt == 3 ? k_prolog_gemm<3> : k_prolog_gemm<4>;
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kPlThreads), 0, st, a, m0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_prolog_norm, dim3((unsigned)a.rows), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace sa
