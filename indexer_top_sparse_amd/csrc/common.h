// Device helpers shared by the gfx950 kernels: MFMA wrappers, bf16 packing, order-preserving
// float keys, block-wide scans and the per-sequence cross-workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define SA_LDS __attribute__((address_space(3)))

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate. Lane l holds
// A[l%16][8*(l/16) + e], B[8*(l/16) + e][l%16] (e = 0..7) and D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32). Lane l holds A[l%32][8*(l/32) + e], B[8*(l/32) + e][l%32]
// and D[8*j + 4*(l/32) + i][l%32] in register 4*j + i.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16) += A(16x128) * B(128x16) on E4M3 codes with one E8M0 scale per row (A) or column
// (B) and 32-entry block of k (v_mfma_scale_f32_16x16x128_f8f6f4). Lane l holds row / column
// l%16: its first 16 code bytes (lo) are k = 16*(l/16) + j, the next 16 (hi) are
// k = 64 + 16*(l/16) + j. The low byte of a lane's scale word is the E8M0 exponent of
// (row / column l%16, block l/16). D is laid out as for mfma16x16x32.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_mx16x16x128(u32x4 alo, u32x4 ahi, uint32_t sa, u32x4 blo,
                                                  u32x4 bhi, uint32_t sb, f32x4 c) {
    const i32x8 a = {(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3],
                     (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
    const i32x8 b = {(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3],
                     (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// fp32 -> OCP E4M3 code: round to nearest, ties to even, saturating at +-448; the sign bit
// follows the sign of y (so -0 and negatives that round to zero give 0x80). Magnitudes below
// the smallest normal (2^-6) are multiples of 2^-9; above it the fp32 mantissa is rounded to 3
// bits and a carry moves to the next binade by itself.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.f);
    const uint32_t b = __float_as_uint(a);
    const uint32_t cn = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);  // normal
    const uint32_t cs = (uint32_t)rintf(a * 512.f);                                // subnormal
    return (a < 0.015625f ? cs : cn) | sign;
}

// MX block exponent from the bit pattern of the block's largest magnitude (bf16, sign cleared):
// floor(log2) of a normal value minus 8 (the exponent of E4M3's largest power of two), clamped
// to [-127, 127]. Zero and subnormal maxima give -127.
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bf16) {
    return max(-127, min(127, (int)(amax_bf16 >> 7) - 127 - 8));
}

// two fp32 -> two bf16 in one word (v_cvt_pk_bf16_f32: round to nearest even), lo first
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four E4M3 codes (one 32-bit word, byte 0 first) -> four bf16 (two words), two codes per
// instruction (v_cvt_scalef32_pk_bf16_fp8 with scale 1). Every E4M3 value, subnormals included,
// is exact in bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t codes) {
    const bf16x2v lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.f, false);
    const bf16x2v hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Order-preserving map float -> uint32 (larger float <=> larger key). -0 maps like +0. Key 0
// only arises from NaN patterns, so it doubles as the "no candidate" marker.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max(x, 0) in one instruction: a float with the sign bit set is a negative int32, so the
// integer max with 0 maps every negative value (and -0) to +0 and keeps the rest. fmaxf would
// first canonicalise x (a second v_max), which MFMA results never need.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Combine each lane's value with the one 32 lanes away (v_permlane32_swap with itself yields
// both halves' values in every lane; the results are identical in the two lanes of a pair).
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// Inclusive prefix sum over the 64 lanes of a wave.
// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips): shifts by 1, 2, 4
// and 8 lanes inside each row of 16 (a lane without a source adds 0), then row r adds the last
// lane of row r - 1 (rows 1 and 3), then lane 31 (rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Sum over the 64 lanes, the same in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}

// Exclusive prefix sum across the block (NT threads); `scratch` needs NT/64 + 1 words.
// Returns the exclusive prefix and stores the block total in *total. Contains barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *scratch,
                                                    uint32_t *total) {
    constexpr int NWV = NT / 64;
    const uint32_t incl = wave_incl_scan(v);
    __syncthreads();
    if (lane_id() == 63) scratch[wave_id()] = incl;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
        const uint32_t s = scratch[i];
        base += (i < wave_id()) ? s : 0u;
        tot += s;
    }
    *total = tot;
    return base + incl - v;
}

// Two exclusive prefix sums across the block at once (one pair of barriers); `scratch` needs
// 2 NT/64 words. Returns the prefix of v; *excl_u gets the prefix of u, *total_v (and *total_u if
// given) the block totals.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan2(uint32_t v, uint32_t u, uint32_t *scratch,
                                                     uint32_t *total_v, uint32_t *excl_u,
                                                     uint32_t *total_u = nullptr) {
    constexpr int NWV = NT / 64;
    const uint32_t iv = wave_incl_scan(v), iu = wave_incl_scan(u);
    __syncthreads();
    if (lane_id() == 63) {
        scratch[wave_id()] = iv;
        scratch[NWV + wave_id()] = iu;
    }
    __syncthreads();
    uint32_t bv = 0, bu = 0, tv = 0, tu = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
        const uint32_t sv = scratch[i], su = scratch[NWV + i];
        bv += (i < wave_id()) ? sv : 0u;
        bu += (i < wave_id()) ? su : 0u;
        tv += sv;
        tu += su;
    }
    *total_v = tv;
    if (total_u) *total_u = tu;
    *excl_u = bu + iu - u;
    return bv + iv - v;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, then meets the
// other waves. Unlike __syncthreads() it does not wait for outstanding global loads, so a
// global->LDS prefetch into another buffer stays in flight across it. The signal fences keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave are
// outstanding (expcnt and lgkmcnt left at their maxima).
__host__ __device__ constexpr int vmcnt_imm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// LDS barrier for use right after an explicit s_waitcnt on vector memory: waits for this
// wave's LDS operations, then meets the other waves.
__device__ __forceinline__ void full_barrier_lds_only_after_wait() { lds_barrier(); }

// The same after all of this wave's global loads (including global->LDS copies) landed.
__device__ __forceinline__ void full_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- cross-workgroup barrier
// Workgroups that share one sequence meet here. The launch never holds more workgroups than the
// device keeps resident at once, so all of them become resident once earlier work has drained.
// All data the workgroups exchange (histograms, counts) is written and
// read only with device-scope atomic operations, which are performed at the device coherence
// point rather than in a per-XCD L2; so no cache-wide fence is needed. Ordering comes from
// waiting until every atomic this workgroup issued has completed (s_waitcnt) before arriving,
// and from reading shared data only after every arrival has been observed.
// `count` only grows during a launch: the j-th barrier (j = 1, 2, ...) of a group of n
// workgroups is passed once count reaches j n, so the last arrival itself releases the others
// (no reset and no second atomic on the way). `j` is the caller's barrier number, advanced
// here; only thread 0's copy is used. The caller's leave step returns count to 0 for the next
// launch (the last of the n workgroups to leave does it).
// A bounded spin keeps every wave finite: after spin_limit polls bit 0 of *err is set and the
// call returns false. The caller then marks its group as failed, and the group's last workgroup
// to leave writes a defined failure result.
__device__ __forceinline__ bool group_barrier(uint32_t *count, uint32_t n, uint32_t *err,
                                              uint32_t &j, uint32_t spin_limit) {
    __shared__ int s_ok;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's atomics and stores have been performed
    __syncthreads();
    ++j;
    if (threadIdx.x == 0) {
        int ok = 1;
        const uint32_t target = j * n;
        const uint32_t arrived =
            __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        if (arrived < target) {
            uint32_t spins = 0;
            while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > spin_limit) {
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    break;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_agent(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane j's
// bytes land at LDS byte address lds_base + 16 j; lds_base must be the same in every lane.
// Written as inline asm on purpose: for the builtin the compiler treats every later LDS read as
// dependent on all copies in flight (it waits for vmcnt(0)), which leaves one tile in flight.
// Callers wait for their own copies with an explicit s_waitcnt vmcnt and keep no other
// vector-memory operation in flight meanwhile (the compiler does not count these copies).
// The copy has no destination register, so no register is written after the asm returns.
__device__ __forceinline__ void copy16_to_lds(const void *g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
                 : "memory");
}

// 8-byte store / load at agent scope: performed at the device's coherence point, so data
// exchanged between workgroups on different XCDs (whose L2 caches are not coherent) is seen
// by the reader once the writer's arrival at a group_barrier has been observed.
__device__ __forceinline__ void st_agent_u64(void *p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent_u64(const void *p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte global load that the compiler keeps as one dwordx4.
__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// The same with the nontemporal hint, for data read exactly once per launch (a streamed key
// cache): it does not displace reused lines from the caches, and streams of such loads over
// randomly placed pages reach a higher HBM read rate than plain loads.
__device__ __forceinline__ u32x4 ldg16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

}  // namespace sa
