// kernels.h - the decode-step kernels for gfx950 (MI355X).
//
// Every contraction of the step is an HBM-bound matrix-vector / small-matrix
// product: weight rows are the 16-row A operand of v_mfma_f32_16x16x32_bf16,
// tokens are its 16 B columns.  The step is four launches (five with an f32
// router):
//   k_dense_in : router logits, latent-down z = W_ld x and shared gate/up
//                (all contract over the hidden size H against x); epilogues:
//                sigmoid + bias keys, z, shared SwiGLU.  The router tiles come
//                first and the top-k + routing metadata run inside this kernel
//                while the latent and shared rows stream.
//   k_w13      : active experts' MXFP4 gate/up rows, fused dequantisation,
//                SwiGLU epilogue -> expert activation a.
//   k_w2       : active experts' MXFP4 down rows; each result is weighted and
//                added into the latent combine ylat.
//   k_out      : latent-up W_lu ylat plus shared-down S2 ash, one bf16 RNE.
//
// Work decomposition.  A workgroup is 8 waves.  It covers RW row groups of
// 32 weight rows (two 16-row MFMA tiles) for one group of token columns; the
// KW = 8 / RW waves of a row group split the reduction dimension K into equal
// slices of SPC 128-element steps and their partial tiles are summed through
// LDS in slice order.  No wave of the hot loops synchronises with another
// workgroup; cross-workgroup communication is limited to the routing (one
// release per router tile and per token) and the f32 atomic adds of the
// expert combine.
//
// Operands.  x is bf16 and enters the MFMA as is (16 tokens per column group).
// The f32 intermediates z, a, ylat and ash are carried as hi = bf16(v) and
// lo = bf16(v - hi) (z, a and ash stored that way by their producers, ylat
// split while it is loaded); hi and lo occupy two adjacent columns of
// the same MFMA (8 tokens per column group) and the two column sums are added
// afterwards, which keeps f32-grade precision at one MFMA per K slice.
//
// K layout within one 128-element step: lane group g = lane/16 owns the 32
// consecutive elements [32g, 32g+32) of the step, one MX block for MXFP4 rows
// (16 code bytes, one scale byte), and feeds them to four MFMAs of 8 elements
// each; the activation operand is read with the same layout, so the
// permutation of K cancels in the dot product.
#pragma once

#include "device_common.h"
#include "routing.h"
#include "step_args.h"

namespace moe {

constexpr int kWG = 8;              // waves per workgroup of the step kernels
constexpr int kWGThreads = kWG * kWave;
constexpr int kXcds = 8;            // XCDs of MI355X; workgroup i runs on XCD i % 8

// ---------------------------------------------------------------------------
// Operand loads
// ---------------------------------------------------------------------------

// bf16 column operand of one step (x).  Lanes without a token read a valid
// row (the caller points them at one) and drop the value, so no load sits
// under a lane-dependent branch.
__device__ __forceinline__ void load_cols_bf16(const uint16_t *X, bool valid, int s,
                                               u32x4 (&rb)[4]) {
    const uint16_t *p = X + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 v = ld16(p + 8 * j);
        rb[j] = valid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
}

// f32 column operand of one step, delivered as the hi (part 0) or lo (part 1)
// bf16 half of each value.
__device__ __forceinline__ uint32_t pack_part(float a, float b, int part) {
    uint32_t h, l;
    split_hl2(a, b, h, l);
    return part ? l : h;
}

__device__ __forceinline__ void load_cols_f32(const float *X, bool valid, int part, int s,
                                              u32x4 (&rb)[4]) {
    const float *p = X + (size_t)s * kKStep;
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ldf4(p + 4 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 a = v[2 * j], b = v[2 * j + 1];
        const u32x4 w = {pack_part(a[0], a[1], part), pack_part(a[2], a[3], part),
                         pack_part(b[0], b[1], part), pack_part(b[2], b[3], part)};
        rb[j] = valid ? w : (u32x4){0u, 0u, 0u, 0u};
    }
}

// ---------------------------------------------------------------------------
// Chunk loops (SPC steps, compile-time, straight-line)
// ---------------------------------------------------------------------------

// The loops below issue every load of a group of steps before the first MFMA
// that consumes one, and keep the scheduler from moving them apart: left
// alone, the compiler recycles the operand registers between the loads of a
// step and serialises several memory round trips per step.
__device__ __forceinline__ void fence_schedule() { __builtin_amdgcn_sched_barrier(0); }

// One 16-row bf16 tile: lane (r = l%16, g = l/16) loads row r's 64 bytes at
// elements [32g, 32g+32) of step s.
__device__ __forceinline__ void load_tile_bf16(const uint16_t *A, int s, u32x4 (&ra)[4]) {
    const uint16_t *p = A + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = ld_weight16(p + 8 * j);
}

__device__ __forceinline__ void mfma_tile(const u32x4 (&ra)[4], const u32x4 (&rb)[4], f32x4 &acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma(as_bf16x8(ra[j]), as_bf16x8(rb[j]), acc);
}

// acc += bf16 tile A . bf16 columns X over steps [s0, s1), two steps (8 KB of
// weights per wave) in flight at a time.
__device__ __forceinline__ void dense_chunk_x(const uint16_t *A, const uint16_t *X, bool valid,
                                              int s0, int s1, f32x4 &acc) {
    int s = s0;
#pragma unroll 1
    for (; s + 1 < s1; s += 2) {
        u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
        load_tile_bf16(A, s, ra0);
        load_tile_bf16(A, s + 1, ra1);
        load_cols_bf16(X, valid, s, rb0);
        load_cols_bf16(X, valid, s + 1, rb1);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
        mfma_tile(ra1, rb1, acc);
    }
    if (s < s1) {
        u32x4 ra0[4], rb0[4];
        load_tile_bf16(A, s, ra0);
        load_cols_bf16(X, valid, s, rb0);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
    }
}

// Output kernel: K runs over [0, L) against lat_up and ylat (f32, split into
// hi/lo while loading), then over [0, Is) against sh_w2 and the shared
// activation (already stored as hi/lo bf16 rows); step s < Ls selects the
// first pair.
struct TwoSource {
    const uint16_t *Aa;
    const float *Xa;  // K in [0, L)
    const uint16_t *Ab;
    const uint16_t *Xb;  // K in [0, Is): the lane's hi or lo row
    int Ls;              // L / 128
};

__device__ __forceinline__ void load_two(const TwoSource &t, bool valid, int part, int s,
                                         u32x4 (&ra)[4], u32x4 (&rb)[4]) {
    if (s < t.Ls) {
        load_tile_bf16(t.Aa, s, ra);
        load_cols_f32(t.Xa, valid, part, s, rb);
    } else {
        load_tile_bf16(t.Ab, s - t.Ls, ra);
        load_cols_bf16(t.Xb, valid, s - t.Ls, rb);
    }
}

__device__ __forceinline__ void dense_chunk_out(const TwoSource &t, bool valid, int part, int s0,
                                                int s1, f32x4 &acc) {
    int s = s0;
#pragma unroll 1
    for (; s + 1 < s1; s += 2) {
        u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
        load_two(t, valid, part, s, ra0, rb0);
        load_two(t, valid, part, s + 1, ra1, rb1);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
        mfma_tile(ra1, rb1, acc);
    }
    if (s < s1) {
        u32x4 ra0[4], rb0[4];
        load_two(t, valid, part, s, ra0, rb0);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
    }
}

// ---------------------------------------------------------------------------
// Workgroup split-K reduction
// ---------------------------------------------------------------------------

// Waves w = rg*KW + kw.  Each writes its partial tile to LDS; after the
// barrier the wave with kw == 0 of each row group sums its group's KW slices
// in slice order and returns true (the leader).  The caller issues the
// barrier that ends the unit before LDS is reused.
__device__ __forceinline__ bool reduce_k1(float *s_red, int wave, int kw, int KW, f32x4 &acc) {
    const int lane = lane_id();
    stf4(s_red + (wave * kWave + lane) * 4, acc);
    __syncthreads();
    if (kw != 0) return false;
    if (KW > 1) {
        acc = zero4();
        for (int j = 0; j < KW; ++j) acc += ldf4(s_red + ((wave + j) * kWave + lane) * 4);
    }
    return true;
}

struct Role {
    int wave, KW, RW, rg, kw;
};

// Dense kernels with several column groups (token groups) read the same
// weight tile once per group.  Unit u runs on XCD u % 8 (workgroups are
// dealt to the eight XCDs in turn), so the groups of one tile group get units
// u = 8 (ncg q' + cg) + x: the same XCD x, issued back to back, and the
// repeated reads hit that XCD's L2.  Units past the last tile group idle.
__device__ __forceinline__ int dense_units(int n_t, int RW, int ncg) {
    const int tgroups = (n_t + RW - 1) / RW;
    return ((tgroups + kXcds - 1) / kXcds) * kXcds * ncg;
}
__device__ __forceinline__ void dense_unit(int u, int ncg, int &cg, int &tg) {
    const int x = u % kXcds, q = u / kXcds;
    cg = q % ncg;
    tg = (q / ncg) * kXcds + x;
}

__device__ __forceinline__ Role role_of(int KW) {
    Role r;
    r.wave = wave_index();
    r.KW = KW;
    r.RW = kWG / KW;
    r.rg = r.wave / KW;
    r.kw = r.wave % KW;
    return r;
}

// ---------------------------------------------------------------------------
// Kernel 0 (f32 router only): logits, scores and keys with plain f32 FMAs.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kBlock) k_router_f32(const StepArgs a) {
    __shared__ RouteLds s_route;
    __shared__ int s_last;
    const int wave = wave_index();
    const int lane = lane_id();
    for (int e = blockIdx.x * kWavesPerBlock + wave; e < a.E; e += gridDim.x * kWavesPerBlock) {
        const float *row = a.router_w32 + (size_t)e * a.H;
        for (int b = 0; b < a.B; ++b) {
            const uint16_t *xb = a.x + (size_t)b * a.H;
            float acc = 0.f;
            for (int h = lane; h < a.H; h += kWave) acc = fmaf(row[h], bf16_val(xb[h]), acc);
            acc = wave_sum(acc);
            if (lane == 0) {
                const float s = sigmoidf_(acc);
                store_agent(a.score + (size_t)b * kMaxExperts + e, s);
                store_agent(a.key + (size_t)b * kMaxExperts + e, s + (a.bias ? a.bias[e] : 0.f));
            }
        }
    }
    // One arrival per workgroup, once the stores of all of its waves have
    // completed.
    wait_vm_all();
    __syncthreads();
    if (wave == 0) {
        const bool last = wave_publish(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u;
        if (lane == 0) s_last = last;
    }
    __syncthreads();
    if (s_last) route_step(route_args(a), &s_route, kWavesPerBlock);
}

// ---------------------------------------------------------------------------
// Kernel 1: router + latent-down + shared gate/up over x.
// ---------------------------------------------------------------------------

// Tiles of 16 rows, in this order: router (E/16), latent-down (L/16), shared
// (Is/8: gate rows 8p..8p+7 and up rows 8p..8p+7 in one tile, so SwiGLU pairs
// D rows i and 8+i, held by lanes l and l+32).
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_dense_in(const StepArgs a) {
    __shared__ RouteLds s_route;
    __shared__ float s_red[kWG * kWave * 4];
    __shared__ int s_last;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const Role ro = role_of(a.kw_in);
    if (threadIdx.x == 0) s_last = 0;
    // The latent combine accumulates into ylat with atomics later in the step.
    for (int i = (blockIdx.x * kWGThreads + threadIdx.x) * 4; i < a.B * a.L;
         i += gridDim.x * kWGThreads * 4)
        stf4(a.ylat + i, zero4());
    const int n_rt = a.n_r16, n_lt = a.L >> 4, n_st = a.Is >> 3;
    const int n_t = n_rt + n_lt + n_st;
    const int ncg = (a.B + 15) >> 4;
    const int units = dense_units(n_t, ro.RW, ncg);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int cg, tg;
        dense_unit(u, ncg, cg, tg);
        const int t = tg * ro.RW + ro.rg;
        const bool active = t < n_t;
        const int tt = active ? t : 0;
        int kind;
        const uint16_t *A;
        if (tt < n_rt) {
            kind = 0;
            A = a.router_w + (size_t)(16 * tt + n) * a.H;
        } else if (tt < n_rt + n_lt) {
            kind = 1;
            A = a.lat_down + (size_t)(16 * (tt - n_rt) + n) * a.H;
        } else {
            kind = 2;
            const int p = tt - n_rt - n_lt;
            A = a.sh_w13 + (size_t)((n < 8 ? 0 : a.Is) + 8 * p + (n & 7)) * a.H;
        }
        const int b = 16 * cg + n;
        const bool valid = b < a.B;
        const uint16_t *X = a.x + (size_t)(valid ? b : 0) * a.H + 32 * g;
        f32x4 acc = zero4();
        if (active)
            dense_chunk_x(A + 32 * g, X, valid, ro.kw * a.spc_in, (ro.kw + 1) * a.spc_in, acc);
        const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
        if (leader && active) {
            if (kind == 0) {
                const int e = 16 * tt + 4 * g;
                if (valid) {
                    const f32x4 bv = a.bias ? ldf4(a.bias + e) : zero4();
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float sv = sigmoidf_(acc[i]);
                        store_agent(a.score + (size_t)b * kMaxExperts + e + i, sv);
                        store_agent(a.key + (size_t)b * kMaxExperts + e + i, sv + bv[i]);
                    }
                }
                if (wave_publish(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u &&
                    lane == 0)
                    s_last = 1;
            } else if (kind == 1) {
                if (valid) {
                    uint16_t *dst = a.zhl + (size_t)b * 2 * a.L + 16 * (tt - n_rt) + 4 * g;
                    store_hl4(dst, dst + a.L, acc);
                }
            } else {
                f32x4 up;
#pragma unroll
                for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
                if (valid && g < 2) {
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[i], up[i]);
                    uint16_t *dst = a.ashhl + (size_t)b * 2 * a.Is + 8 * (tt - n_rt - n_lt) + 4 * g;
                    store_hl4(dst, dst + a.Is, v);
                }
            }
        }
        __syncthreads();
        if (s_last) {  // this workgroup completed the router: route the step
            route_step(route_args(a), &s_route, kWG);
            __syncthreads();
            if (threadIdx.x == 0) s_last = 0;
        }
    }
}

// ---------------------------------------------------------------------------
// Expert kernels (2 and 3): shared structure
// ---------------------------------------------------------------------------
//
// A workgroup serves one column unit (one expert, up to 8 of its tokens) and
// 8 row tiles of that expert, one per wave; each wave runs the whole
// reduction length K of its tile, so no partial sums cross waves.  K is taken
// in chunks of S steps (S <= 16, 2048 elements).  Per chunk a wave issues all
// of its MXFP4 code and scale loads at once (S x 16 B of codes per lane), the
// workgroup copies the unit's activation rows for the chunk straight from
// global memory into LDS, and the MFMAs run once everything has landed.  The
// only round trips a workgroup waits on are its unit record, then one chunk
// of weights.

// LDS image of a unit's activation operand for one chunk: row n = 2j + part
// (pair j's hi or lo values), 16 S chunks of 16 bytes (8 bf16) per row; chunk
// q of row n is stored at position q ^ n of its row (n < 16 flips only the
// low four bits of q, so a chunk stays in its 16-chunk block), which puts the
// 16 rows of one MFMA operand read on distinct LDS banks.
template <int S>
struct Stage {
    static constexpr int kRowChunks = 16 * S;
    static constexpr int kChunks = 16 * kRowChunks;  // 16 rows
};

// Wave-cooperative copy of rows 0 .. 2 nt - 1 of the operand for K range
// [k0, k0 + 128 S): source row (j, part) starts at src + row_of(j) * 2 K +
// part * K + k0 (elements).  Every wave takes every 8th 64-chunk block; each
// lane moves one 16-byte chunk with a direct global -> LDS load, which lands
// at the block base + 16 * lane.
template <int S, typename RowOf>
__device__ __forceinline__ void stage_operand(uint16_t *s_b, const uint16_t *src, int K, int k0,
                                              int nt, RowOf row_of) {
    const int lane = lane_id(), wave = wave_index();
    const int total = 2 * nt * Stage<S>::kRowChunks;
    for (int c0 = 64 * wave; c0 < total; c0 += 64 * kWG) {
        const int c = c0 + lane;
        const int n = c / Stage<S>::kRowChunks, st = c % Stage<S>::kRowChunks;
        const int q = st ^ (n & 15);
        const int j = n >> 1, part = n & 1;
        const uint16_t *g = src + ((size_t)row_of(j) * 2 + part) * K + k0 + 8 * q;
        if (c < total) __builtin_amdgcn_global_load_lds(g, s_b + 8 * c0, 16, 0, 0);
    }
}

// Operand of MFMA jj at step s for lane (row n_eff, lane group g).
template <int S>
__device__ __forceinline__ bf16x8 stage_read(const uint16_t *s_b, int n_eff, int g, int s, int jj) {
    const int q = 16 * s + ((4 * g + jj) ^ n_eff);
    return as_bf16x8(*(const u32x4 *)(s_b + 8 * (n_eff * Stage<S>::kRowChunks + q)));
}

// One chunk of one MXFP4 tile row per lane: codes (16 B per step: lane
// group g's 32-element block) and the step's four scale bytes.
template <int S>
struct Fp4Chunk {
    u32x4 code[S];
    uint32_t scale[S];
};

// Scale bytes of the chunk (four per step, lane group g uses byte g).
template <int S>
__device__ __forceinline__ void load_fp4_scales(const uint8_t *sc, Fp4Chunk<S> &w) {
    if constexpr (S % 4 == 0) {
#pragma unroll
        for (int m = 0; m < S / 4; ++m) {
            const u32x4 v = ld_weight16(sc + 16 * m);
#pragma unroll
            for (int i = 0; i < 4; ++i) w.scale[4 * m + i] = v[i];
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) w.scale[s] = ld_weight4(sc + 4 * s);
    }
}

// Codes of the chunk: S loads of 16 bytes, 64 bytes apart (never merged),
// issued in step order, so that step s waits only for the loads up to its
// own.
template <int S>
__device__ __forceinline__ void load_fp4_codes(const uint8_t *q, Fp4Chunk<S> &w) {
#pragma unroll
    for (int s = 0; s < S; ++s) w.code[s] = ld_weight16(q + 64 * s);
}

// Number of weight loads of a chunk that may still be in flight when the
// staging copies have landed.  For S % 4 == 0 the scales are S / 4 loads of 16
// bytes (never merged) issued after the copies together with the codes;
// otherwise they are issued before the copies (the compiler may merge 4-byte
// loads, so their count is not fixed) and only the S code loads follow.
template <int S>
constexpr int loads_after_staging() {
    return S % 4 == 0 ? S + S / 4 : S;
}

// Waits until this wave's staging copies have landed while the weight loads
// issued after them may still be in flight: vector memory loads complete in
// issue order.
template <int S>
__device__ __forceinline__ void wait_staging() {
    constexpr int n = loads_after_staging<S>();
    static_assert(n <= 63, "vmcnt field");
    // s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Workgroup barrier after wait_staging: LDS holds every wave's copy once all
// waves pass it.  A plain barrier, without the memory fence of
// __syncthreads, which would also wait for the weight loads still in flight.
__device__ __forceinline__ void staged_barrier() {
    fence_schedule();
    __builtin_amdgcn_s_barrier();
    fence_schedule();
}

// The MFMAs of one chunk; the activation operand of step s + 1 is read from
// LDS while step s multiplies.  The compiler waits for each step's weight
// registers just before their first use.
template <int S>
__device__ __forceinline__ void mfma_fp4_chunk(const Fp4Chunk<S> &w, const uint16_t *s_b,
                                               int n_eff, int g, f32x4 &acc) {
    const int sh = 8 * g;
    bf16x8 b[2][4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) b[0][jj] = stage_read<S>(s_b, n_eff, g, 0, jj);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) b[(s + 1) & 1][jj] = stage_read<S>(s_b, n_eff, g, s + 1, jj);
        }
        const float f = e8m0_scale((w.scale[s] >> sh) & 0xFFu);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc = mfma(fp4x8_to_bf16(w.code[s][jj], f), b[s & 1][jj], acc);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: expert gate/up (MXFP4) + SwiGLU.
// ---------------------------------------------------------------------------

// Tile t of expert e: gate rows 8t .. 8t+7 (MFMA rows 0-7) and up rows
// I + 8t .. I + 8t + 7 (MFMA rows 8-15), so lanes l and l + 32 hold a gate and
// its up value.  Output: the activation of each pair as hi/lo bf16 rows.
template <int S>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_w13(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_b[8 * Stage<S>::kChunks];
    const int lane = lane_id(), n = lane & 15, g = lane >> 4, wave = wave_index();
    const int j = n >> 1, part = n & 1;
    const int NC = min(a.meta[M_N_COLS], a.ncols_cap);  // never beyond the records
    const int OT = a.I >> 3;
    const int TG = (OT + kWG - 1) / kWG;
    const int nchunk = a.L / (kKStep * S);
    const size_t qrow = a.L / 2, srow = a.L / 32;
    bool reuse = false;  // s_b holds a previous chunk
    for (int u = blockIdx.x; u < NC * TG; u += gridDim.x) {
        const int c = u / TG;
        const int t = (u % TG) * kWG + wave;
        const bool active = t < OT;
        const int recw = a.cu_rec[c * kRecWords + (lane & 31)];
        const int e = (int)readlane((uint32_t)recw, R_EXPERT);
        const int nt = (int)readlane((uint32_t)recw, R_COUNT);
        const int p0 = (int)readlane((uint32_t)recw, R_PAIR0);
        const int n_eff = j < nt ? n : part;
        const size_t r = (size_t)e * 2 * a.I + (n < 8 ? 0 : a.I) + 8 * (active ? t : 0) + (n & 7);
        const uint8_t *qp = a.w13_q + r * qrow + 16 * g;
        const uint8_t *sp = a.w13_s + r * srow;
        f32x4 acc = zero4();
        for (int ch = 0; ch < nchunk; ++ch) {
            // Every wave loads and multiplies (a wave past the last tile
            // reads tile 0 again and drops its result), which keeps the
            // load sequence free of branches: the compiler then waits for
            // each step's own loads only.  The staging copies go first, so
            // that the barrier below waits for them alone.
            if (reuse) __syncthreads();  // every wave is done with s_b
            reuse = true;
            Fp4Chunk<S> w;
            if constexpr (S % 4 != 0) load_fp4_scales<S>(sp + (size_t)ch * S * 4, w);
            fence_schedule();
            stage_operand<S>(s_b, a.zhl, a.L, ch * S * kKStep, nt,
                             [&](int jj) { return __shfl(recw, R_TOKEN + jj); });
            fence_schedule();
            if constexpr (S % 4 == 0) load_fp4_scales<S>(sp + (size_t)ch * S * 4, w);
            load_fp4_codes<S>(qp + (size_t)ch * S * 64, w);
            fence_schedule();
            wait_staging<S>();
            staged_barrier();
            mfma_fp4_chunk<S>(w, s_b, n_eff, g, acc);
        }
        acc = add_pair_column(acc);
        f32x4 up;
#pragma unroll
        for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
        if (active && j < nt && part == 0 && g < 2) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[i], up[i]);
            uint16_t *dst = a.acthl + (size_t)(p0 + j) * 2 * a.I + 8 * t + 4 * g;
            store_hl4(dst, dst + a.I, v);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 3: expert down (MXFP4) + weighted combine in latent space.
// ---------------------------------------------------------------------------

// Tile t of expert e: latent rows 16t .. 16t+15; the routing weight of each
// pair scales its column before the f32 atomic add into ylat.
template <int S>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_w2(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_b[8 * Stage<S>::kChunks];
    const int lane = lane_id(), n = lane & 15, g = lane >> 4, wave = wave_index();
    const int j = n >> 1, part = n & 1;
    const int NC = min(a.meta[M_N_COLS], a.ncols_cap);  // never beyond the records
    const int OT = a.L >> 4;
    const int TG = (OT + kWG - 1) / kWG;
    const int nchunk = a.I / (kKStep * S);
    const size_t qrow = a.I / 2, srow = a.I / 32;
    bool reuse = false;  // s_b holds a previous chunk
    for (int u = blockIdx.x; u < NC * TG; u += gridDim.x) {
        const int c = u / TG;
        const int t = (u % TG) * kWG + wave;
        const bool active = t < OT;
        const int recw = a.cu_rec[c * kRecWords + (lane & 31)];
        const int e = (int)readlane((uint32_t)recw, R_EXPERT);
        const int nt = (int)readlane((uint32_t)recw, R_COUNT);
        const int p0 = (int)readlane((uint32_t)recw, R_PAIR0);
        const int jc = j < nt ? j : 0;
        const int tok_j = __shfl(recw, R_TOKEN + jc);
        const float w_j = __int_as_float(__shfl(recw, R_WEIGHT + jc));
        const int n_eff = j < nt ? n : part;
        const size_t r = (size_t)e * a.L + 16 * (active ? t : 0) + n;
        const uint8_t *qp = a.w2_q + r * qrow + 16 * g;
        const uint8_t *sp = a.w2_s + r * srow;
        f32x4 acc = zero4();
        for (int ch = 0; ch < nchunk; ++ch) {
            // Every wave loads and multiplies (a wave past the last tile
            // reads tile 0 again and drops its result), which keeps the
            // load sequence free of branches: the compiler then waits for
            // each step's own loads only.  The staging copies go first, so
            // that the barrier below waits for them alone.
            if (reuse) __syncthreads();  // every wave is done with s_b
            reuse = true;
            Fp4Chunk<S> w;
            if constexpr (S % 4 != 0) load_fp4_scales<S>(sp + (size_t)ch * S * 4, w);
            fence_schedule();
            stage_operand<S>(s_b, a.acthl, a.I, ch * S * kKStep, nt,
                             [&](int jj) { return p0 + jj; });
            fence_schedule();
            if constexpr (S % 4 == 0) load_fp4_scales<S>(sp + (size_t)ch * S * 4, w);
            load_fp4_codes<S>(qp + (size_t)ch * S * 64, w);
            fence_schedule();
            wait_staging<S>();
            staged_barrier();
            mfma_fp4_chunk<S>(w, s_b, n_eff, g, acc);
        }
        acc = add_pair_column(acc);
        if (active && j < nt && part == 0) {
            float *dst = a.ylat + (size_t)tok_j * a.L + 16 * t + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + i, w_j * acc[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 4: latent-up + shared-down, bf16 output.
// ---------------------------------------------------------------------------

// Output tiles cover RT = out_rows <= 16 rows (MFMA rows past RT repeat the
// tile's last row and are dropped), chosen so that the tiles split evenly
// over the compute units.
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_out(const StepArgs a) {
    __shared__ float s_red[kWG * kWave * 4];
    // The router counter of the dense input kernel is cleared here, where no
    // wave of the step can touch it any more.
    if (blockIdx.x == 0 && threadIdx.x == 0) a.gctr[G_ROUTER_DONE] = 0u;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const Role ro = role_of(a.kw_out);
    const int RT = a.out_rows;
    const int ncg = (a.B + 7) >> 3;
    const int n_t = (a.H + RT - 1) / RT;
    const int units = dense_units(n_t, ro.RW, ncg);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int cg, tg;
        dense_unit(u, ncg, cg, tg);
        const int t = tg * ro.RW + ro.rg;
        const bool active = t < n_t;
        const int b = 8 * cg + col;
        const bool valid = b < a.B;
        const int bb = valid ? b : 0;
        const int h0 = RT * (active ? t : 0);
        const size_t h = min(h0 + min(n, RT - 1), a.H - 1);
        TwoSource ts;
        ts.Aa = a.lat_up + h * a.L + 32 * g;
        ts.Xa = a.ylat + (size_t)bb * a.L + 32 * g;
        ts.Ab = a.sh_w2 + h * a.Is + 32 * g;
        ts.Xb = a.ashhl + ((size_t)bb * 2 + part) * a.Is + 32 * g;
        ts.Ls = a.L / kKStep;
        f32x4 acc = zero4();
        if (active)
            dense_chunk_out(ts, valid, part, ro.kw * a.spc_out, (ro.kw + 1) * a.spc_out, acc);
        const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
        if (leader && active) {
            acc = add_pair_column(acc);
            if (valid && part == 0) {
                uint16_t *dst = a.out + (size_t)b * a.H;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;
                    if (r < RT && h0 + r < a.H) dst[h0 + r] = (uint16_t)bf16_rne(acc[i]);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Support kernels (set-up and inspection; not part of the step).
// ---------------------------------------------------------------------------

__global__ void k_fill_u32(uint32_t *p, size_t n, uint32_t v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// MXFP4 -> f32 with the routine the expert kernels use (8 elements / thread).
__global__ void k_dequant(const uint8_t *q, const uint8_t *s, int64_t n, float *out) {
    const int64_t i = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * 8;
    if (i >= n) return;
    const uint32_t codes = *(const uint32_t *)(q + i / 2);
    const bf16x8 v = fp4x8_to_bf16(codes, e8m0_scale(s[i / 32]));
#pragma unroll
    for (int j = 0; j < 8; ++j) out[i + j] = (float)v[j];
}

struct DebugArgs {
    float *score, *key, *z, *act, *ylat, *ash;
    int32_t *n_active;
};

__global__ void k_debug_export(const StepArgs a, const DebugArgs d) {
    const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t nE = (size_t)a.B * a.E, nL = (size_t)a.B * a.L, nS = (size_t)a.B * a.Is;
    const size_t nA = (size_t)a.B * a.k * a.I;
    for (size_t i = tid; i < nE; i += stride) {
        const size_t j = (i / a.E) * kMaxExperts + i % a.E;
        if (d.score) d.score[i] = a.score[j];
        if (d.key) d.key[i] = a.key[j];
    }
    for (size_t i = tid; i < nL; i += stride) {
        const size_t b = i / a.L, c = i % a.L;
        const uint16_t *zr = a.zhl + b * 2 * a.L;
        if (d.z) d.z[i] = bf16_val(zr[c]) + bf16_val(zr[a.L + c]);
        if (d.ylat) d.ylat[i] = a.ylat[i];
    }
    for (size_t i = tid; i < nS; i += stride) {
        const size_t b = i / a.Is, c = i % a.Is;
        const uint16_t *r = a.ashhl + b * 2 * a.Is;
        if (d.ash) d.ash[i] = bf16_val(r[c]) + bf16_val(r[a.Is + c]);
    }
    for (size_t i = tid; i < nA; i += stride) {
        if (!d.act) break;
        const size_t slot = i / a.I, c = i % a.I;
        const uint16_t *ar = a.acthl + (size_t)a.pair_of_slot[slot] * 2 * a.I;
        d.act[i] = bf16_val(ar[c]) + bf16_val(ar[a.I + c]);
    }
    if (tid == 0 && d.n_active) d.n_active[0] = a.meta[M_N_ACTIVE];
}

}  // namespace moe
