// Row-wise Top-K over scores in HBM: the selection step of Prefill, whose scores are
// materialised, and of sa_topk. Ties at the threshold go to the lower positions and the indices
// come out in ascending order. The Top-K filtering operator of "Engineering Path for Day-0
// Adaptation of Trillion-Scale Sparse Models on Domestic AI Accelerators" §3.1.
//  - Rows of up to 65536 scores: k_topk_rows_1r reads each row once (a sampled lower bound of
//    the threshold, the candidates at or above it listed as the row streams, an exact selection
//    over them).
//  - Longer rows, and rows whose candidates do not fit its list: the streaming selection, radix
//    passes over the row (digits of 11/11/10 bits, stopping as soon as the threshold bin is
//    taken whole); when the first digit's threshold bin and above fit in LDS, one more read
//    collects them and the selection ends there.
#include "common.h"
#include "kernels.h"

namespace sa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkUnroll = 8;   // histogram passes: keys per thread whose loads are in flight together
constexpr int kTkPer = 16;     // emission: consecutive keys per thread per round
constexpr int kTkList = 7168;  // LDS list of (key, position) for the one-more-read path (56 KiB)

// The selection of one row by a workgroup of kTkThreads threads, reading the row from HBM (in
// shared memory: hist[2048], scan[2 kTkWaves + 1], res[4], lkey and lpos[CAP]).
// Block-uniform; contains barriers.
template <int CAP>
__device__ __forceinline__ void topk_row_stream(const TopkArgs &a, int row, uint32_t *hist,
                                                uint32_t *scan, uint32_t *res, uint32_t *lkey,
                                                int32_t *lpos) {
    const int tid = threadIdx.x;
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
        if (pass == 0 && res[1] + res[2] <= (uint32_t)CAP) {
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

__global__ __launch_bounds__(kTkThreads) void k_topk_rows(TopkArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t scan[2 * kTkWaves + 1];
    __shared__ uint32_t res[4];
    __shared__ uint32_t lkey[kTkList];
    __shared__ int32_t lpos[kTkList];
    topk_row_stream<kTkList>(a, blockIdx.x, hist, scan, res, lkey, lpos);
}

// A value the compiler may not take apart or move across other such values (asm statements keep
// their program order).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// ------------------------------------------------- rows of up to 65536 keys, one read
// Several 512-thread workgroups share a CU, so that the selection work of some overlaps the
// loads of others, and the row is read from HBM once:
//  1. A sample of 4096 positions spread over the row, loaded ahead of it, gives a lower bound of the
//     threshold: the lower edge of the 22-bit bin (two 11-bit digits) holding its ks-th largest
//     key, ks a quarter above the sample's share of k, plus 16. It is found while the row's
//     first loads are in flight.
//  2. The row streams through registers in groups of 16 scores per thread, kTqDepth groups in
//     flight; every score whose key reaches the bound goes with its position to an LDS list
//     (per group, one slot range per wave from one LDS atomic). The listed set is
//     closed upwards in the key order, so when it holds at least k positions it holds the Top-K.
//  3. The exact Top-K of the list by (key, position) composites, radix passes in LDS, and the
//     emission through a bitmap of the row (positions 128 t .. 128 t + 127 belong to thread t).
// Rows shorter than 8192, with k above an eighth of the row, or whose list is too short or too
// long take the streaming selection. VEC = 4 reads 16 bytes per load (the row start 16-byte
// aligned), VEC = 1 four bytes; both with the nontemporal hint (the row is read once).
// PERCU resident workgroups per CU: four (k up to 2048: a list of 4000 candidates, 64 registers,
// two groups in flight) or two (larger k: 7168 candidates, three groups in flight).
constexpr int kTqT = kTkThreads;             // 512 threads, the streaming selection's block
constexpr int kTqMax = 65536;                // longest row
constexpr int kTqGroups = kTqMax / (16 * kTqT);  // groups of 16 scores per thread
constexpr int kTqSample = 8;                 // sampled positions per thread (tq_sample_pos)
constexpr int kTqSmallK = 2048;              // largest k of the four-per-CU form
static_assert(kTqGroups == 8 && kTqMax / 128 == kTqT && kTqSample * kTqT * 16 == kTqMax, "");
template <int PERCU>
struct TqCfg {
    static constexpr int kList = PERCU == 4 ? 4000 : 7168;  // candidates
    static constexpr int kDepth = PERCU == 4 ? 2 : 3;       // groups in flight
};

// sampled position i (0..7) of thread t: the first 32 positions of every block of 512 (whole
// 128-byte lines, evenly spread over the row, so that a row whose large scores gather in one
// region, as recent positions may, is sampled there too)
__device__ __forceinline__ int tq_sample_pos(int i, int t) {
    return 8192 * i + 512 * (t >> 5) + (t & 31);
}

// position of score e (0..15) of group g, thread t
template <int VEC>
__device__ __forceinline__ int tq_pos(int g, int e, int t) {
    return VEC == 4 ? 2048 * (4 * g + (e >> 2)) + 4 * t + (e & 3)
                    : 1024 * (8 * g + (e >> 1)) + 512 * (e & 1) + t;
}

template <int VEC, int PERCU>
__global__ __launch_bounds__(kTqT, PERCU * kTqT / 256) void k_topk_rows_1r(TopkArgs a) {
    constexpr int kTqList = TqCfg<PERCU>::kList, kTqDepth = TqCfg<PERCU>::kDepth;
    __shared__ uint32_t hist[2048];  // also the emission's bitmap of the row
    __shared__ uint32_t scan[2 * kTkWaves + 1];
    __shared__ uint32_t res[4];
    __shared__ uint32_t lkey[kTqList];
    __shared__ int32_t lpos[kTqList];
    __shared__ uint32_t lcount;
    const int row = blockIdx.x, tid = threadIdx.x;
    int seq, qoff, qlen;
    row_info(a.q_indptr, a.num_seqs, row, seq, qoff, qlen);
    const int64_t pos_q = (int64_t)a.ctx_lens[seq] - qlen + qoff;
    const int n = (int)min(pos_q + 1, a.ld);  // n <= kTqMax (the host checks ld)
    const uint32_t k_eff = (uint32_t)min(a.k, max(n, 0));
    const float *sc = a.scores + (int64_t)row * a.ld;
    int32_t *out = a.idx + (int64_t)row * a.k;

    int len = 0;
    if (k_eff > 0 && n >= 8192 && 8 * (int64_t)k_eff <= n) {
        // ---- the sample's loads, then the row's first groups (every load issued, clamped to
        //      the last visible position; positions past the row are masked when used). The
        //      thread index passes through an opaque copy per group and every group's last
        //      use through one as well: the compiler keeps those in program order, so it can
        //      neither hoist later groups' loads nor sink a group's work past them.
        float smp[kTqSample];
#pragma unroll
        for (int i = 0; i < kTqSample; ++i)
            smp[i] = __builtin_nontemporal_load(&sc[min(tq_sample_pos(i, tid), n - 1)]);
        float gb[kTqDepth][16];
        auto issue = [&](int g, float (&b)[16]) {
            const int t = (int)opaque_u32((uint32_t)threadIdx.x);
            if constexpr (VEC == 4) {
                const int last = (n - 1) >> 2;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 v = ldg16_stream(sc + 4 * min(kTqT * (4 * g + i) + t, last));
#pragma unroll
                    for (int e = 0; e < 4; ++e) b[4 * i + e] = __uint_as_float(v[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) b[e] = __builtin_nontemporal_load(&sc[min(tq_pos<1>(g, e, t), n - 1)]);
            }
        };
#pragma unroll
        for (int g = 0; g < kTqDepth - 1; ++g) issue(g, gb[g]);
        // ---- 1. the bound, from two 11-bit digits of the sample's keys (LDS-only barriers: the
        //      row's loads stay in flight): the sample's ks-th largest key lies in bin b1 of the
        //      first digit and then in bin b2 of the second, and the bound is that bin's lower edge
        const int w = wave_id();
        uint32_t skey[kTqSample];
#pragma unroll
        for (int i = 0; i < kTqSample; ++i) {
            const uint32_t k = float_key(smp[i]);
            skey[i] = tq_sample_pos(i, tid) < n ? k : 0u;  // 0: outside the row (or the NaN keyed 0)
        }
        // block-wide suffix scan of hist (thread t owns bins 2047 - 4 t - j, j < 4): the bin
        // holding the need-th largest entry goes to res[0], the count above it to res[1]
        auto find_bin = [&](uint32_t need) {
            uint32_t hv[4], csum = 0;
            const int top = 2048 - 4 * tid - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hv[j] = hist[top - j];
                csum += hv[j];
            }
            const uint32_t incl = wave_incl_scan(csum);
            if (lane_id() == 63) scan[w] = incl;
            lds_barrier();
            uint32_t run = incl - csum;
#pragma unroll
            for (int i = 0; i < kTkWaves; ++i) run += i < w ? scan[i] : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (run < need && run + hv[j] >= need) {
                    res[0] = (uint32_t)(top - j);
                    res[1] = run;
                }
                run += hv[j];
            }
        };
        for (int i = tid; i < 2048; i += kTqT) hist[i] = 0u;
        if (tid == 0) {
            lcount = 0u;
            res[0] = 0u;
            res[1] = 0u;
        }
        uint32_t mine_s = 0;
#pragma unroll
        for (int i = 0; i < kTqSample; ++i) mine_s += skey[i] != 0u ? 1u : 0u;
        const uint32_t ws = wave_incl_scan(mine_s);
        if (lane_id() == 63) scan[kTkWaves + w] = ws;
        lds_barrier();
        uint32_t ns = 0;  // sampled keys inside the row
#pragma unroll
        for (int i = 0; i < kTkWaves; ++i) ns += scan[kTkWaves + i];
#pragma unroll
        for (int i = 0; i < kTqSample; ++i)
            if (skey[i] != 0u) atomicAdd(&hist[skey[i] >> 21], 1u);
        lds_barrier();
        const uint32_t need_s =
            (uint32_t)min<int64_t>(ns, ((int64_t)k_eff * ns + n - 1) / n * 5 / 4 + 16);
        find_bin(need_s);
        lds_barrier();
        const uint32_t b1 = res[0], above1 = res[1];
        for (int i = tid; i < 2048; i += kTqT) hist[i] = 0u;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kTqSample; ++i)
            if (skey[i] != 0u && (skey[i] >> 21) == b1) atomicAdd(&hist[(skey[i] >> 10) & 2047u], 1u);
        lds_barrier();
        find_bin(need_s - above1);
        lds_barrier();
        // keys at or above the lower edge of that bin (never 0: positions past the row and the
        // one NaN pattern whose key is 0 stay out)
        const uint32_t bound = max((b1 << 21) | (res[0] << 10), 1u);
        // ---- 2. the row, group by group, listing the keys at or above the bound
#pragma unroll
        for (int g = 0; g < kTqGroups; ++g) {
            if (g + kTqDepth - 1 < kTqGroups)
                issue(g + kTqDepth - 1, gb[(g + kTqDepth - 1) % kTqDepth]);
            const int t = (int)opaque_u32((uint32_t)threadIdx.x);
            uint32_t key[16], mine = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // opaque: the group's work cannot move above the next group's loads
                const uint32_t k = float_key(__uint_as_float(opaque_u32(__float_as_uint(gb[g % kTqDepth][e]))));
                key[e] = tq_pos<VEC>(g, e, t) < n ? k : 0u;
                mine += key[e] >= bound ? 1u : 0u;
            }
            // one slot range per wave: an LDS atomic by the last lane, broadcast
            const uint32_t wincl = wave_incl_scan(mine);
            uint32_t base = 0;
            if (__builtin_amdgcn_readlane((int)wincl, 63) != 0) {
                if (lane_id() == 63) base = atomicAdd(&lcount, wincl);
                base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63);
            }
            uint32_t dst = base + wincl - mine;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (key[e] >= bound) {
                    if (dst < (uint32_t)kTqList) {
                        lkey[dst] = key[e];
                        lpos[dst] = tq_pos<VEC>(g, e, t);
                    }
                    ++dst;
                }
            }
            dst = opaque_u32(dst);
        }
        lds_barrier();
        const uint32_t c_tot = lcount;
        if (c_tot >= k_eff && c_tot <= (uint32_t)kTqList) len = (int)c_tot;
        __syncthreads();  // every thread has read lcount
    }

    if (len == 0) {  // block-uniform
        topk_row_stream<kTqList>(a, row, hist, scan, res, lkey, lpos);
        return;
    }
    // ---- 3. exact Top-K of the list by composites (key << 32 | ~position: a larger composite
    //      is a larger score or, for equal scores, a lower position), radix passes in LDS
    uint64_t pre = 0;
    int pb = 0;
    uint32_t lneed = k_eff;
    while (pb < 64) {
        const int nbits = min(11, 64 - pb);
        const int shift = 64 - pb - nbits;
        const int nb = 1 << nbits;
        for (int i = tid; i < 2048; i += kTqT) hist[i] = 0u;
        __syncthreads();
        for (int j = tid; j < len; j += kTqT) {
            const uint64_t c = ((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)lpos[j];
            if (pb == 0 || (c >> (64 - pb)) == pre)
                atomicAdd(&hist[(uint32_t)(c >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        uint32_t hv[4], csum = 0;
        const int top = nb - 4 * tid - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hv[j] = top - j >= 0 ? hist[top - j] : 0u;
            csum += hv[j];
        }
        if (tid == 0) res[0] = 0u;
        uint32_t tot;
        uint32_t run = block_excl_scan<kTqT>(csum, scan, &tot);
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
        pre = (pre << nbits) | res[0];
        pb += nbits;
        const bool whole = res[2] == lneed;  // always true once all 64 bits are used
        __syncthreads();
        if (whole) break;
    }
    // ---- emission in position order through a bitmap of the row (in the histogram's words, free
    //      since the last pass's final barrier): the taken positions set their bits; thread t
    //      owns words 4 t .. 4 t + 3, and one block scan of their population counts gives each
    //      word the number of taken positions before it. A taken entry's output slot is that
    //      count plus the taken positions before it in its own word. The index row is staged in
    //      LDS (over the list's keys, which are not read again) and written out coalesced.
    const uint64_t thr = pb < 64 ? pre << (64 - pb) : pre;
    uint32_t *bits = hist;
    uint32_t *wpre = reinterpret_cast<uint32_t *>(lpos) + kTqList - 2048;  // per-word counts
    int32_t *stage = reinterpret_cast<int32_t *>(lkey);
    // (k_eff <= len <= kTqList, so the index row fits over the keys)
    static_assert(kTqList >= 2048, "the word counts fit in the list's positions");
#pragma unroll
    for (int i = 0; i < 4; ++i) bits[4 * tid + i] = 0u;
    __syncthreads();
    for (int j = tid; j < len; j += kTqT) {
        const int pos = lpos[j];
        if ((((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)pos) >= thr)
            atomicOr(&bits[pos >> 5], 1u << (pos & 31));
    }
    __syncthreads();
    {
        uint32_t wv[4], c[4], cnt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wv[i] = bits[4 * tid + i];
            c[i] = (uint32_t)__popc(wv[i]);
            cnt += c[i];
        }
        uint32_t tot;
        uint32_t run = block_excl_scan<kTqT>(cnt, scan, &tot);
        // the word counts go to the list's last 2048 position slots, so every listed position is
        // read into registers first
        int32_t pl[kTqList / kTqT + 1];
#pragma unroll
        for (int q = 0; q < kTqList / kTqT + 1; ++q) {
            const int j = tid + q * kTqT;
            pl[q] = j < len ? lpos[j] : -1;
        }
        __syncthreads();  // every listed position is in registers
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wpre[4 * tid + i] = run;
            run += c[i];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kTqList / kTqT + 1; ++q) {
            const int pos = pl[q];
            if (pos < 0) continue;
            const uint32_t wd = bits[pos >> 5], bit = 1u << (pos & 31);
            if (wd & bit) {
                const uint32_t slot = wpre[pos >> 5] + (uint32_t)__popc(wd & (bit - 1u));
                if (slot < k_eff) stage[slot] = pos;
            }
        }
    }
    __syncthreads();
    for (int j = tid; j < (int)k_eff; j += kTqT) out[j] = stage[j];
    for (int j = (int)k_eff + tid; j < a.k; j += kTqT) out[j] = -1;
}

hipError_t launch_topk_rows(const TopkArgs &a, int rows, hipStream_t st) {
    if (a.ld <= kTqMax) {
        const bool v4 = a.ld % 4 == 0 && reinterpret_cast<uintptr_t>(a.scores) % 16 == 0;
        const bool small_k = a.k <= kTqSmallK;
        const void *kern = v4 ? (small_k ? reinterpret_cast<const void *>(&k_topk_rows_1r<4, 4>)
                                         : reinterpret_cast<const void *>(&k_topk_rows_1r<4, 2>))
                              : (small_k ? reinterpret_cast<const void *>(&k_topk_rows_1r<1, 4>)
                                         : reinterpret_cast<const void *>(&k_topk_rows_1r<1, 2>));
        void *args[] = {const_cast<TopkArgs *>(&a)};
        return hipLaunchKernel(kern, dim3(rows), dim3(kTqT), args, 0, st);
    } else {
        hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(kTkThreads), 0, st, a);
    }
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
