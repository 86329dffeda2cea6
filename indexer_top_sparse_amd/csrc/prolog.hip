// Indexer prolog on gfx950: the three projections that feed the indexer (query, key, head
// weights) as one grid of MFMA tiles, then the key's LayerNorm.
//
// "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei
// Ascend CANN Architecture" (CANN) §2.2: Q projection with K normalization, and Q quantization
// with the head-weight projection, run as independent work before the indexer. Here the
// independent projections share one launch (their tiles fill the device together instead of
// three streams each holding part of it); Q quantization happens inside the MXFP8 indexer.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kPlThreads = 256;  // 4 waves; each takes a quarter of a tile's contraction

// Contraction slice of a key / head-weight tile: 512 entries of the hidden input, or 256 / 128
// when 512 does not divide its width.
__host__ __device__ inline int pl_slice(int d_model) {
    return d_model % 512 == 0 ? 512 : (d_model % 256 == 0 ? 256 : 128);
}

// Tiles, in launch order: key and head-weight tiles (kPlCols of the dim + heads output columns
// x one slice of the hidden input; their partial sums go to the workspace), then query tiles
// (kPlCols output columns x the whole query input, written as bf16).
constexpr int kPlCT = 2;              // 16-column MFMA tiles per wave
constexpr int kPlCols = 16 * kPlCT;  // output columns of a workgroup

struct PlJob {
    bool query;
    int n0, nmax, K, slice;
    const uint16_t *x, *w;  // activations [rows][ldx] and the weight row of column n0, at the job's k0
    int ldx;
};

__device__ __forceinline__ PlJob pl_job(const PrologArgs &a, int t) {
    const int nkw = (a.dim + a.heads + kPlCols - 1) / kPlCols, sw = pl_slice(a.d_model),
              ns = a.d_model / sw;
    if (t < nkw * ns) {
        const int c = t % nkw, sl = t / nkw, n0 = kPlCols * c;
        // columns [0, dim) are key columns (rows of W_k), [dim, dim + heads) head-weight columns
        // (rows of W_w); dim is a multiple of kPlCols, so a tile holds one kind
        const bool key = n0 < a.dim;
        const uint16_t *w = key ? a.w_k + (size_t)n0 * a.d_model
                                : a.w_w + (size_t)(n0 - a.dim) * a.d_model;
        return {false, n0, key ? a.dim : a.dim + a.heads, sw, sl, a.x + (size_t)sl * sw,
                w + (size_t)sl * sw, a.d_model};
    }
    t -= nkw * ns;
    return {true, kPlCols * t, a.heads * a.dim, a.d_q, 0, a.x_q,
            a.w_q + (size_t)kPlCols * t * a.d_q, a.d_q};
}

// y[m][n] = sum_k x[m][k] * W[n][k] over the job's contraction for MT 16-row tiles from row m0
// and its kPlCols columns. MFMA 16x16x32: A = x (lane l: row l%16, k = 8(l/16)..), B = W^T (lane
// l: column l%16 of a 16-column tile, the same k); one activation fragment feeds kPlCT MFMAs.
// Every 16-row x 32-k piece is loaded coalesced (lane l: row l/4, 16 bytes l%4: four requests
// of 64 contiguous bytes per 16 lanes, instead of sixteen of 16 bytes in the MFMA lane order)
// and transposed into the MFMA order through the wave's own 1 KiB of LDS (XOR-swizzled, so both
// sides are free of bank conflicts). Rows and columns past the ends read the last valid row
// (loads stay unconditional) and are not stored. Every tile of the grid reads the same
// activation rows, so each tile walks its contraction from a different starting k-step: the
// requests of concurrent tiles then spread over the L2 channels.
template <int MT>
__global__ __launch_bounds__(kPlThreads) void k_prolog_gemm(PrologArgs a, int m0) {
    __shared__ f32x4 red[4][kPlCT][MT][64];
    __shared__ u32x4 tr[4][64];  // per-wave transpose area
    const PlJob j = pl_job(a, blockIdx.x);
    const int l = lane_id(), w = wave_id(), g = l >> 4;
    const int kq = j.K / 4;  // this wave's quarter of the contraction, a multiple of 32
    const int steps = kq / 32;
    // coalesced load order: lane l takes row l/4, bytes 16 (l%4) .. of the 64 of a k-step
    const int lr = l >> 2, lc = l & 3;
    const uint16_t *wp[kPlCT];
#pragma unroll
    for (int ct = 0; ct < kPlCT; ++ct) {
        const int nrow = min(j.n0 + 16 * ct + lr, j.nmax - 1) - j.n0;
        wp[ct] = j.w + (size_t)nrow * j.ldx + (size_t)w * kq + 8 * lc;
    }
    const uint16_t *xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xp[mt] = j.x + (size_t)min(m0 + 16 * mt + lr, a.rows - 1) * j.ldx + (size_t)w * kq + 8 * lc;
    // 16-byte unit of (row r, chunk c) in the transpose area: 4 rows per 256-byte line, the
    // chunk index XOR-ed with the line index
    auto unit = [](int r, int c) { return (r >> 2) * 16 + (r & 3) * 4 + (c ^ ((r >> 2) & 3)); };
    u32x4 *tw = tr[w];
    const int wu = unit(lr, lc), ru = unit(l & 15, g);
    auto frag = [&](u32x4 v) {  // coalesced piece -> MFMA fragment (this wave's LDS only)
        tw[wu] = v;
        return tw[ru];
    };
    f32x4 acc[kPlCT][MT];
#pragma unroll
    for (int ct = 0; ct < kPlCT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // k-steps in groups of U, two groups in flight; every group issues the same loads (a group
    // past the end re-reads the last step and multiplies nothing), so each wait is exact
    constexpr int U = 4;
    const int ng = (steps + U - 1) / U;
    const int rot = (int)(blockIdx.x % (unsigned)steps);
    u32x4 b[2][U][kPlCT], xf[2][U][MT];
    auto load = [&](int buf, int grp) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int s = min(grp * U + u, steps - 1) + rot;
            s = 32 * (s >= steps ? s - steps : s);
#pragma unroll
            for (int ct = 0; ct < kPlCT; ++ct) b[buf][u][ct] = ldg16(wp[ct] + s);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xf[buf][u][mt] = ldg16(xp[mt] + s);
        }
    };
    auto mul = [&](int buf, int grp) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (grp * U + u < steps) {
                u32x4 bf[kPlCT], xv[MT];
#pragma unroll
                for (int ct = 0; ct < kPlCT; ++ct) bf[ct] = frag(b[buf][u][ct]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xv[mt] = frag(xf[buf][u][mt]);
#pragma unroll
                for (int ct = 0; ct < kPlCT; ++ct)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[ct][mt] = mfma16x16x32(xv[mt], bf[ct], acc[ct][mt]);
            }
    };
    load(0, 0);
    for (int grp = 0; grp < ng; grp += 2) {
        load(1, grp + 1);
        mul(0, grp);
        load(0, grp + 2);
        mul(1, grp + 1);
    }
    // sum the four quarters: wave w adds up the (column, row) tiles w, w + 4, ...
#pragma unroll
    for (int ct = 0; ct < kPlCT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[w][ct][mt][l] = acc[ct][mt];
    __syncthreads();
    const int ncols = a.dim + a.heads;
    for (int t = w; t < kPlCT * MT; t += 4) {
        const int ct = t / MT, mt = t % MT;
        f32x4 s = red[0][ct][mt][l];
#pragma unroll
        for (int v = 1; v < 4; ++v) s += red[v][ct][mt][l];
        const int col = j.n0 + 16 * ct + (l & 15);
        if (col >= j.nmax) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * mt + 4 * g + i;
            if (m >= a.rows) continue;
            if (j.query) a.q_out[(size_t)m * j.nmax + col] = (uint16_t)(pack_bf16x2(s[i], 0.f) & 0xFFFFu);
            else a.part[((size_t)j.slice * a.rows + m) * ncols + col] = s[i];
        }
    }
}

// Per row: key and head-weight columns summed over the slices in slice order; the head weights
// are stored, the key goes through the LayerNorm: mean, then the mean of squared deviations,
// (y - mean) / sqrt(var + eps) * gamma + beta, rounded to bf16. One thread per column.
__global__ __launch_bounds__(256) void k_prolog_norm(PrologArgs a) {
    __shared__ float s_red[2][4];
    const int row = blockIdx.x, c = threadIdx.x, l = lane_id(), w = wave_id();
    const int ncols = a.dim + a.heads, ns = a.d_model / pl_slice(a.d_model);
    // the slices' partial sums, eight loads in flight, added in slice order
    float y = 0.f;
    const float *pp = a.part + (size_t)row * ncols + min(c, ncols - 1);
    const size_t stride = (size_t)a.rows * ncols;
    for (int s0 = 0; s0 < ns; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pp[(size_t)min(s0 + u, ns - 1) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < ns) y += v[u];
    }
    if (c >= ncols) y = 0.f;
    if (c >= a.dim && c < ncols) a.w_out[(size_t)row * a.heads + (c - a.dim)] = y;
    const bool key = c < a.dim;
    // block sums over the key columns (dim <= 128: waves 0 and 1)
    auto block_sum = [&](float v, int slot) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (l == 0) s_red[slot][w] = v;
        __syncthreads();
        return s_red[slot][0] + s_red[slot][1] + s_red[slot][2] + s_red[slot][3];
    };
    const float mu = block_sum(key ? y : 0.f, 0) / (float)a.dim;
    const float d = key ? y - mu : 0.f;
    const float var = block_sum(d * d, 1) / (float)a.dim;
    const float inv = 1.f / sqrtf(var + a.eps);
    if (key)
        a.k_out[(size_t)row * a.dim + c] = (uint16_t)(pack_bf16x2(d * inv * a.gamma[c] + a.beta[c], 0.f) & 0xFFFFu);
}

size_t prolog_workspace_bytes(int rows, int dim, int heads, int d_model) {
    return (size_t)(d_model / pl_slice(d_model)) * rows * (dim + heads) * 4;
}

hipError_t launch_prolog(const PrologArgs &a, hipStream_t st) {
    const int tiles = ((a.dim + a.heads + kPlCols - 1) / kPlCols) * (a.d_model / pl_slice(a.d_model)) +
                      (a.heads * a.dim + kPlCols - 1) / kPlCols;
    for (int m0 = 0; m0 < a.rows; m0 += 64) {
        const int mt = min(4, (a.rows - m0 + 15) / 16);
        auto kern = mt == 1 ? k_prolog_gemm<1> : mt == 2 ? k_prolog_gemm<2>
                  : mt == 3 ? k_prolog_gemm<3> : k_prolog_gemm<4>;
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kPlThreads), 0, st, a, m0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_prolog_norm, dim3((unsigned)a.rows), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace sa
