// Row-wise Top-K over scores in HBM (the unfused selection used by Prefill and by tests):
// one workgroup per query row, radix select on order-preserving keys (three digits of
// 11/11/10 bits, stopping as soon as the threshold bin is taken whole), then an ordered
// emission that keeps ascending positions and gives ties at the threshold to the lower
// positions. When the keys of the first digit's threshold bin and above fit in LDS, one more
// read collects them and the selection ends there (two reads of the row instead of three). "Top-K filtering ... custom operator" of "Engineering Path for Day-0 Adaptation of
// Trillion-Scale Sparse Models on Domestic AI Accelerators" §3.1.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkUnroll = 8;   // histogram passes: keys per thread whose loads are in flight together
constexpr int kTkPer = 16;     // emission: consecutive keys per thread per round
constexpr int kTkList = 7168;  // LDS list of (key, position) for the one-more-read path (56 KiB)

__global__ __launch_bounds__(kTkThreads) void k_topk_rows(TopkArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t scan[2 * kTkWaves + 1];
    __shared__ uint32_t res[4];
    __shared__ uint32_t lkey[kTkList];
    __shared__ int32_t lpos[kTkList];
    const int row = blockIdx.x, tid = threadIdx.x;
    int seq, qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int64_t pos_q = (int64_t)a.ctx_lens[seq] - qlen + qoff;
    const int n = (int)min(pos_q + 1, a.ld);
    const float *sc = a.scores + (int64_t)row * a.ld;
    int32_t *out = a.idx + (int64_t)row * a.k;
    const uint32_t k_eff = (uint32_t)min(a.k, max(n, 0));

    uint32_t prefix = 0, need = k_eff;
    int pbits = 0;
    bool exact = false;
    uint32_t listed = 0;  // > 0: the selection finishes on the LDS list
    for (int pass = 0; pass < 3 && need > 0; ++pass) {
        const int bits = pass < 2 ? 11 : 10;
        const int shift = 32 - pbits - bits;
        const int nb = 1 << bits;
        for (int i = tid; i < 2048; i += kTkThreads) hist[i] = 0u;
        __syncthreads();
        // coalesced keys, kTkUnroll loads in flight per thread: issued unconditionally (clamped
        // to the last key; the opaque copies keep them out of branches), then masked
        for (int i0 = tid; i0 < n; i0 += kTkUnroll * kTkThreads) {
            uint32_t kk[kTkUnroll];
#pragma unroll
            for (int u = 0; u < kTkUnroll; ++u) kk[u] = float_key(sc[min(i0 + u * kTkThreads, n - 1)]);
#pragma unroll
            for (int u = 0; u < kTkUnroll; ++u) {
                asm volatile("" : "+v"(kk[u]));
                const uint32_t k = kk[u];
                if (i0 + u * kTkThreads >= n) continue;
                if (pbits && (k >> (32 - pbits)) != prefix) continue;
                atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
            }
        }
        __syncthreads();
        uint32_t hv[4], csum = 0;
        const int top = nb - 4 * tid - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hv[j] = top - j >= 0 ? hist[top - j] : 0u;
            csum += hv[j];
        }
        uint32_t tot;
        uint32_t run = block_excl_scan<kTkThreads>(csum, scan, &tot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (run < need && run + hv[j] >= need) {
                res[0] = (uint32_t)(top - j);
                res[1] = run;
                res[2] = hv[j];
            }
            run += hv[j];
        }
        __syncthreads();
        need -= res[1];
        prefix = (prefix << bits) | res[0];
        pbits += bits;
        if (res[2] == need) {
            exact = true;
            break;
        }
        // the keys above the first threshold bin plus those in it fit in LDS: one more read
        // collects them, and the rest happens there
        if (pass == 0 && res[1] + res[2] <= (uint32_t)kTkList) {
            listed = res[1] + res[2];
            break;
        }
        __syncthreads();
    }

    if (listed > 0) {
        // ---- collect the keys of the threshold bin and above, in position order: rounds of
        //      kTkPer consecutive keys per thread, one scan per round
        const uint32_t T = prefix;  // 11 bits
        uint32_t lbase = 0;
        for (int base = 0; base < n; base += kTkPer * kTkThreads) {
            const int i0 = base + kTkPer * tid;
            uint32_t keys[kTkPer];
#pragma unroll
            for (int j = 0; j < kTkPer; ++j) keys[j] = float_key(sc[min(i0 + j, n - 1)]);
            uint32_t mine = 0;
#pragma unroll
            for (int j = 0; j < kTkPer; ++j) {
                asm volatile("" : "+v"(keys[j]));  // keeps the loads above out of branches
                mine += (i0 + j < n && (keys[j] >> 21) >= T) ? 1u : 0u;
            }
            uint32_t tot;
            uint32_t dst = lbase + block_excl_scan<kTkThreads>(mine, scan, &tot);
#pragma unroll
            for (int j = 0; j < kTkPer; ++j)
                if (i0 + j < n && (keys[j] >> 21) >= T) {
                    lkey[dst] = keys[j];
                    lpos[dst] = i0 + j;
                    ++dst;
                }
            lbase += tot;
        }
        __syncthreads();
        // ---- exact threshold among the bin's keys: radix passes over the composites
        //      (key << 32 | ~position; a larger composite is a larger score or, for equal
        //      scores, a lower position) in LDS
        uint64_t pre = T;
        int pb = 11;
        uint32_t lneed = need;
        const int len = (int)listed;
        for (;;) {
            const int bits = min(11, 64 - pb);
            const int shift = 64 - pb - bits;
            const int nb = 1 << bits;
            for (int i = tid; i < 2048; i += kTkThreads) hist[i] = 0u;
            __syncthreads();
            for (int j = tid; j < len; j += kTkThreads) {
                const uint64_t c = ((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)lpos[j];
                if ((c >> (64 - pb)) == pre) atomicAdd(&hist[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
            }
            __syncthreads();
            uint32_t hv[4], csum = 0;
            const int top = nb - 4 * tid - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hv[j] = top - j >= 0 ? hist[top - j] : 0u;
                csum += hv[j];
            }
            uint32_t tot;
            uint32_t run = block_excl_scan<kTkThreads>(csum, scan, &tot);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < lneed && run + hv[j] >= lneed) {
                    res[0] = (uint32_t)(top - j);
                    res[1] = run;
                    res[2] = hv[j];
                }
                run += hv[j];
            }
            __syncthreads();
            lneed -= res[1];
            pre = (pre << bits) | res[0];
            pb += bits;
            const bool whole = res[2] == lneed;  // always true once all 64 bits are used
            __syncthreads();
            if (whole) break;
        }
        // ---- emission from the list (already in position order): a key is taken when its
        //      composite reaches the threshold composite, which every key above the bin does
        const uint64_t thr = pre << (64 - pb);
        const int E = (len + kTkThreads - 1) / kTkThreads;
        const int e0 = min(len, tid * E), e1 = min(len, e0 + E);
        uint32_t mine = 0;
        for (int j = e0; j < e1; ++j)
            mine += ((((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)lpos[j]) >= thr) ? 1u : 0u;
        uint32_t tot;
        uint32_t dst = block_excl_scan<kTkThreads>(mine, scan, &tot);
        for (int j = e0; j < e1; ++j)
            if ((((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)lpos[j]) >= thr) {
                if (dst < k_eff) out[dst] = lpos[j];
                ++dst;
            }
    }

    // ordered emission, rounds of kTkPer consecutive keys per thread: keys above the threshold
    // prefix are taken, and keys equal to it are taken in position order while fewer than
    // `need` of them have been (all of them when the threshold bin is taken whole). One scan
    // of (above, equal) counts per round gives every thread its first slot: the keys above
    // before it plus the equal keys taken before it.
    if (k_eff > 0 && listed == 0) {
        const int shb = 32 - pbits;
        const uint32_t need_eq = exact ? 0xFFFFFFFFu : need;
        uint32_t above_base = 0, eq_base = 0;
        for (int base = 0; base < n; base += kTkPer * kTkThreads) {
            const int i0 = base + kTkPer * tid;
            uint32_t keys[kTkPer];
#pragma unroll
            for (int j = 0; j < kTkPer; ++j) keys[j] = float_key(sc[min(i0 + j, n - 1)]);
            uint32_t my_above = 0, my_eq = 0;
#pragma unroll
            for (int j = 0; j < kTkPer; ++j) {
                asm volatile("" : "+v"(keys[j]));
                const bool in = i0 + j < n;
                const uint32_t p = keys[j] >> shb;
                my_above += (in && p > prefix) ? 1u : 0u;
                my_eq += (in && p == prefix) ? 1u : 0u;
            }
            uint32_t tot_above, tot_eq, eq_excl;
            const uint32_t above_excl =
                block_excl_scan2<kTkThreads>(my_above, my_eq, scan, &tot_above, &eq_excl, &tot_eq);
            uint32_t er = eq_base + eq_excl;
            uint32_t dst = above_base + above_excl + min(er, need_eq);
#pragma unroll
            for (int j = 0; j < kTkPer; ++j) {
                if (i0 + j >= n) break;
                const uint32_t p = keys[j] >> shb;
                bool take = p > prefix;
                if (p == prefix) {
                    take = er < need_eq;
                    ++er;
                }
                if (take) {
                    if (dst < k_eff) out[dst] = i0 + j;
                    ++dst;
                }
            }
            above_base += tot_above;
            eq_base += tot_eq;
        }
    }
    for (int j = (int)k_eff + tid; j < a.k; j += kTkThreads) out[j] = -1;
}

hipError_t launch_topk_rows(const TopkArgs &a, int rows, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(kTkThreads), 0, st, a);
    return hipGetLastError();
}

__global__ void k_zero(uint4 *p, size_t n16) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t n16 = bytes / 16;
    if (n16) {
        const size_t want = (n16 + 255) / 256;
        const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
        hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, st, (uint4 *)p, n16);
    }
    return hipGetLastError();
}

}  // namespace sa
