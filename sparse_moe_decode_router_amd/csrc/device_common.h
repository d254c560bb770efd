// device_common.h - gfx950 device helpers shared by the decode-step kernels:
// vector types, bf16 rounding and hi/lo splitting, MXFP4 -> bf16 conversion
// with the E8M0 block scale, the 16x16x32 bf16 MFMA, wave reductions and the
// agent-scope counters used by the routing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_limits.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// f32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// Two f32 -> two bf16 (low half: a), round to nearest even, with the
// packed conversion instruction.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// (a, b) ~= hi + lo with hi = bf16(v), lo = bf16(v - hi) per value; the
// residual of the pair is below 2^-17 |v|.  Both halves as packed bf16 pairs.
__device__ __forceinline__ void split_hl2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = bf16x2_rne(a, b);
    lo = bf16x2_rne(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

// Writes four values as hi and lo bf16 halves (8 bytes each).  Coh: with
// agent-scope stores, for rows that other workgroups of the same launch read
// (the fused step); otherwise plain stores, which a later launch reads.
template <bool Coh>
__device__ __forceinline__ void store_hl4(uint16_t *hi, uint16_t *lo, f32x4 v) {
    uint32_t h0, l0, h1, l1;
    split_hl2(v[0], v[1], h0, l0);
    split_hl2(v[2], v[3], h1, l1);
    const uint64_t hv = (uint64_t)h0 | ((uint64_t)h1 << 32);
    const uint64_t lv = (uint64_t)l0 | ((uint64_t)l1 << 32);
    if constexpr (Coh) {
        __hip_atomic_store((uint64_t *)hi, hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store((uint64_t *)lo, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *(uint64_t *)hi = hv;
        *(uint64_t *)lo = lv;
    }
}

// E8M0 byte -> f32 scale 2^(byte-127) (bytes 1..254).
__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// a power-of-two scale -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float scale) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, f32) += A(16x32) B(32x16).  Lane l supplies A row l%16 and B
// column l%16, eight K values each (lane group l/16 picks which eight); it
// receives D rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// Adds the value of the neighbouring column (lane ^ 1): joins the hi and lo
// column of one token.
__device__ __forceinline__ f32x4 add_pair_column(f32x4 v) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i] + __shfl_xor(v[i], 1);
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}

// Exclusive prefix sum over the wave; *total receives the sum of all lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int *total) {
    const int lane = lane_id();
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(inc, d);
        if (lane >= d) inc += o;
    }
    *total = __shfl(inc, kWave - 1);
    return inc - v;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Publication without cache maintenance.  Data that one workgroup publishes
// to another through a counter is written with agent-scope atomic stores
// (they go through to the agent's point of coherence instead of staying in
// this XCD's L2) and read with agent-scope atomic loads (which do not hit a
// stale line in the reader's caches).  An arrival then only has to wait until
// the wave's own stores have completed before it increments the counter: no
// L2 write-back (release fence) on the writer side, no invalidation
// (acquire fence) on the reader side.
__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte loads through a buffer resource over [base, base + 2 GiB).  Coh:
// with the sc1 cache policy (as agent-scope atomic loads use), which reads
// the agent's coherent copy, for operands another workgroup of the same
// launch wrote; otherwise a plain load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCohAux = 16;  // cache policy bits: sc1
template <bool Coh>
constexpr int cache_aux() {
    return Coh ? kCohAux : 0;
}
__device__ __forceinline__ rsrc_t buf_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7FFFFFFF, 0x00020000);
}
template <bool Coh>
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, cache_aux<Coh>()));
}

// 16-byte store through a buffer resource.  Coh: with the sc1 cache policy
// that agent-scope atomic stores use, for values another workgroup of the
// same launch reads (one 16-byte store per lane instead of two 8-byte atomic
// stores, so a wave writes whole 1 KiB blocks).
template <bool Coh>
__device__ __forceinline__ void buf_st16(rsrc_t r, uint32_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, cache_aux<Coh>());
}

// Waits for every vector memory access of the wave (stores included).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wave-wide fetch-add on an agent-scope counter: lane 0 adds v (the other
// lanes add zero, so the atomic sits under no lane-dependent branch) and the
// old value is returned as a scalar.
__device__ __forceinline__ uint32_t wave_fetch_add(uint32_t *ctr, uint32_t v) {
    const uint32_t add = lane_id() == 0 ? v : 0u;
    const uint32_t old = __hip_atomic_fetch_add(ctr, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return uniform(old);
}

// One arrival of the whole wave on an agent-scope counter after its
// agent-scope stores (see above) have completed; returns the old value.
__device__ __forceinline__ uint32_t wave_publish(uint32_t *ctr) {
    wait_vm_all();
    return wave_fetch_add(ctr, 1u);
}

// Index of the calling wave in its workgroup, as a scalar.
__device__ __forceinline__ int wave_index() { return (int)uniform(threadIdx.x >> 6); }

// Weight streams: read once per step, never written by the step.  Plain
// loads measured faster than non-temporal ones on gfx950 for this stream.
// Everything the step itself produces is read with ordinary loads after a
// kernel boundary or an acquire, never through a path that may run ahead of
// the synchronisation.
__device__ __forceinline__ u32x4 ld_weight16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ uint32_t ld_weight4(const void *p) { return *(const uint32_t *)p; }
__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ f32x4 ldf4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ void stf4(float *p, f32x4 v) { *(f32x4 *)p = v; }

__device__ __forceinline__ float sigmoidf_(float t) { return 1.0f / (1.0f + expf(-t)); }
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace moe
