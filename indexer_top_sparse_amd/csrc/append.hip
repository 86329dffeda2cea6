// Cache append on gfx950: the new tokens' indexer keys and KV rows written into the paged
// caches at their slots, quantized into the caches' formats, and the summaries of the blocks
// that received a token recomputed. One workgroup per new token row; a second launch updates the
// summaries once every row of a block is in place.
//
// Pages cited: "How the Ascend Computing Platform Achieves Same-Day Inference Adaptation for
// Ultra-Large Sparse Models" (SameDay) §3.1 (coarse filtering over block summaries kept in the
// cache); "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on
// Huawei Ascend CANN Architecture" (CANN) §3 (MXFP8 indexer, FP8 KV per 128-entry tile);
// "Engineering Path for Day-0 Adaptation of Trillion-Scale Sparse Models on Domestic AI
// Accelerators" (Domestic) §3.2 (blocked layout: block number + offset).
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kAppThreads = 256;

// position and physical slot of a new token row (the last qlen positions of its sequence)
__device__ __forceinline__ bool append_slot(const AppendArgs &a, int row, int &seq, int &pos,
                                            int64_t &slot) {
    int qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int ctx = a.ctx_lens[seq];
    pos = ctx - qlen + qoff;
    if (pos < 0 || pos >= ctx) return false;
    const int P = 1 << a.lp;
    slot = (int64_t)a.page_table[(int64_t)seq * a.pages_per_seq + (pos >> a.lp)] * P + (pos & (P - 1));
    return true;
}

__device__ __forceinline__ float bf16_at(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

// E4M3 code of x with the scale sigma: the quotient is rounded to fp32 (IEEE division), then to
// E4M3 (nearest, ties to even, saturating)
__device__ __forceinline__ uint8_t e4m3_scaled(float x, float sigma) {
    return (uint8_t)e4m3_rne(__fdiv_rn(x, sigma));
}

__device__ __forceinline__ float sigma_of(uint32_t amax_bits) {
    const float amax = __uint_as_float(amax_bits);
    return amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
}

__global__ __launch_bounds__(kAppThreads) void k_cache_append(AppendArgs a) {
    // magnitude maxima as fp32 bit patterns (non-negative floats order like their bits):
    // [0..7] KV tiles (or [0] the KV row), [8] the indexer row, [12..15] MXFP8 groups
    __shared__ uint32_t s_max[16];
    const int tid = threadIdx.x, row = blockIdx.x;
    int seq, pos;
    int64_t slot;
    if (!append_slot(a, row, seq, pos, slot)) return;
    if (tid < 16) s_max[tid] = 0u;
    __syncthreads();

    // ---- pass 1: maxima of the quantization groups
    const int D = a.idx_dim;
    const uint16_t *ki = a.k_idx_new ? a.k_idx_new + (int64_t)row * D : nullptr;
    if (ki && a.idx_fmt != 0)
        for (int i = tid; i < D; i += kAppThreads) {
            const uint32_t m = __float_as_uint(fabsf(bf16_at(ki, i)));
            atomicMax(&s_max[a.idx_fmt == 1 ? 8 : 12 + i / 32], m);
        }
    const int W = a.heads_kv * a.dim_qk;  // KV row entries
    const int nt = (a.dim_qk + 127) / 128;
    const uint16_t *kn = a.kv_new ? a.kv_new + (int64_t)row * W : nullptr;
    if (kn && a.kv_fmt != 0)
        for (int i = tid; i < W; i += kAppThreads) {
            const uint32_t m = __float_as_uint(fabsf(bf16_at(kn, i)));
            const int g = a.kv_fmt == 1 ? 0 : (i / a.dim_qk) * nt + (i % a.dim_qk) / 128;
            atomicMax(&s_max[g], m);
        }
    __syncthreads();

    // ---- pass 2: stores
    if (ki) {
        if (a.idx_fmt == 0) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(a.idx_keys) + slot * D;
            for (int i = tid; i < D; i += kAppThreads) dst[i] = ki[i];
        } else if (a.idx_fmt == 1) {
            const float sg = sigma_of(s_max[8]);
            uint8_t *dst = a.idx_keys + slot * D;
            for (int i = tid; i < D; i += kAppThreads) dst[i] = e4m3_scaled(bf16_at(ki, i), sg);
            if (tid == 0) a.idx_scale[slot] = sg;
        } else {
            uint8_t *dst = a.idx_keys + slot * D;
            for (int i = tid; i < D; i += kAppThreads) {
                const int x = mx_block_exp(s_max[12 + i / 32] >> 16);  // bf16 bits of the group max
                dst[i] = (uint8_t)e4m3_rne(ldexpf(bf16_at(ki, i), -x));
                if (i % 32 == 0) a.idx_mx[slot * (D / 32) + i / 32] = (uint8_t)(x + 127);
            }
        }
    }
    if (kn) {
        if (a.kv_fmt == 0) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(a.kc) + slot * W;
            for (int i = tid; i < W; i += kAppThreads) dst[i] = kn[i];
            if (a.v_new) {
                const int WV = a.heads_kv * a.dim_v;
                const uint16_t *vn = a.v_new + (int64_t)row * WV;
                uint16_t *dv = reinterpret_cast<uint16_t *>(a.vc) + slot * WV;
                for (int i = tid; i < WV; i += kAppThreads) dv[i] = vn[i];
            }
        } else {
            uint8_t *dst = a.kc + slot * W;
            for (int i = tid; i < W; i += kAppThreads) {
                const int g = a.kv_fmt == 1 ? 0 : (i / a.dim_qk) * nt + (i % a.dim_qk) / 128;
                dst[i] = e4m3_scaled(bf16_at(kn, i), sigma_of(s_max[g]));
            }
            if (a.kv_fmt == 1) {
                if (tid == 0) a.kv_scale[slot] = sigma_of(s_max[0]);
            } else if (tid < a.heads_kv * nt) {
                a.kv_scale[slot * a.heads_kv * nt + tid] = sigma_of(s_max[tid]);
            }
        }
    }
}

// Block summaries: the row that is its block's last new row (the block's last position, or the
// sequence's last) recomputes the block's mean over its valid keys: summed in fp64 in position
// order, divided by the count, rounded to fp32 and then to bf16. Thread d owns entry d.
__global__ __launch_bounds__(128) void k_pool_update(AppendArgs a) {
    const int row = blockIdx.x, d = threadIdx.x;
    int seq, pos;
    int64_t slot;
    if (!append_slot(a, row, seq, pos, slot)) return;
    const int P = 1 << a.lp;
    const int ctx = a.ctx_lens[seq];
    if ((pos & (P - 1)) != P - 1 && pos != ctx - 1) return;
    if (d >= a.idx_dim) return;
    const int first = pos & ~(P - 1);
    const int last = min(first + P - 1, ctx - 1);
    const int64_t page = a.page_table[(int64_t)seq * a.pages_per_seq + (pos >> a.lp)];
    const uint16_t *keys = reinterpret_cast<const uint16_t *>(a.idx_keys);
    const uint16_t *kp = keys + page * P * a.idx_dim + d;  // entry d of the block's first row
    double s = 0.0;
    int t = first;
    // 16 loads in flight, then the additions in position order
    for (; t + 16 <= last + 1; t += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = bf16_at(kp, (int64_t)((t + u) & (P - 1)) * a.idx_dim);
#pragma unroll
        for (int u = 0; u < 16; ++u) s += (double)v[u];
    }
    for (; t <= last; ++t) s += (double)bf16_at(kp, (int64_t)(t & (P - 1)) * a.idx_dim);
    const float f = (float)(s / (double)(last - first + 1));
    const uint32_t u = __float_as_uint(f);
    a.pooled[page * a.idx_dim + d] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Whole-page copies (copy-on-write of shared pages): workgroup (pair, table) copies page src
// of one table to page dst, 4-byte words when the page's bytes allow, else bytes.
__global__ __launch_bounds__(256) void k_copy_pages(PageCopyArgs a) {
    const int pr = blockIdx.x, t = blockIdx.y;
    const int64_t bytes = a.page_bytes[t];
    if (!a.base[t] || bytes == 0) return;
    const int64_t src = a.pairs[2 * pr], dst = a.pairs[2 * pr + 1];
    uint8_t *b = a.base[t];
    if (bytes % 4 == 0) {
        const uint32_t *s = reinterpret_cast<const uint32_t *>(b + src * bytes);
        uint32_t *d = reinterpret_cast<uint32_t *>(b + dst * bytes);
        for (int64_t i = threadIdx.x; i < bytes / 4; i += 256) d[i] = s[i];
    } else {
        for (int64_t i = threadIdx.x; i < bytes; i += 256) b[dst * bytes + i] = b[src * bytes + i];
    }
}

hipError_t launch_copy_pages(const PageCopyArgs &a, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_copy_pages, dim3((unsigned)n, (unsigned)kPageTables), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_cache_append(const AppendArgs &a, int rows, bool pool, hipStream_t st) {
    hipLaunchKernelGGL(k_cache_append, dim3((unsigned)rows), dim3(kAppThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !pool) return e;
    hipLaunchKernelGGL(k_pool_update, dim3((unsigned)rows), dim3(128), 0, st, a);
    return hipGetLastError();
}

}  // namespace sa
