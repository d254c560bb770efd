// kernels.h - the decode-step kernels for gfx950 (MI355X).
//
// Every contraction of the step is an HBM-bound matrix-vector / small-matrix
// product: weight rows are the 16-row A operand of v_mfma_f32_16x16x32_bf16,
// tokens are its 16 B columns.  The step's work comes in units, each run by
// one workgroup of 8 waves:
//   dense-in : router rows, latent-down rows z = W_ld x, shared gate/up rows
//              (all against x); epilogues: sigmoid + bias keys, z, shared
//              SwiGLU; the router units also drive the routing (top-k and
//              the expert lists);
//   w13      : an active expert's MXFP4 gate/up rows for <= 8 of its tokens,
//              SwiGLU -> expert activation a;
//   w2       : an active expert's MXFP4 down rows; weighted, f32 atomic adds
//              into the latent combine ylat;
//   output   : latent-up rows against ylat and shared-down rows against ash,
//              one bf16 rounding.
// The units run either as four launches (k_dense_in, k_w13, k_w2, k_out; an
// f32 router adds k_router_f32) or as one persistent launch (k_step) whose
// workgroups take units from a queue in dependency order and wait on
// completion counters instead of kernel boundaries.
//
// Dense units: RW row groups of 16 rows; the KW = 8 / RW waves of a row group
// split K into equal slices of SPC 128-element steps and sum their partial
// tiles through LDS in slice order.  Expert units: every wave runs the whole
// K of its tile, with the unit's activation rows staged in LDS.
//
// Operands.  x is bf16 and enters the MFMA as is (16 tokens per column group).
// The f32 intermediates z, a, ylat and ash are carried as hi = bf16(v) and
// lo = bf16(v - hi) (z, a and ash stored that way by their producers, ylat
// split while it is loaded); hi and lo occupy two adjacent columns of
// the same MFMA (8 tokens per column group) and the two column sums are added
// afterwards, which keeps f32-grade precision at one MFMA per K slice.  Data
// one unit hands to another within one launch (scores, keys; in the
// persistent kernels also z, a, ash, the shared-down sums and the expert
// records) is written with agent-scope stores and read with coherent (sc1)
// loads, so that it is visible across XCDs without cache maintenance; data
// crossing a kernel boundary uses plain accesses.
//
// K layout within one 128-element step.  MXFP4 rows: lane group g = lane/16
// owns the 32 consecutive elements [32g, 32g+32) of the step, one MX block
// (16 code bytes, one scale byte), and feeds them to four MFMAs of 8
// elements each.  bf16 rows: MFMA j takes elements [32j + 8g, 32j + 8g + 8)
// from lane group g, so each load instruction reads 64 contiguous bytes of a
// row.  The activation operand is read with the layout of its weights, so the
// permutation of K cancels in the dot product.
#pragma once

#include "device_common.h"
#include "routing.h"
#include "step_args.h"

namespace moe {

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
        const u32x4 v = ld16(p + 32 * j);
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

// Column operands an earlier unit wrote, read through a buffer resource
// (Coh: coherent loads, the writer being a unit of the same launch): `off` is
// the byte offset of the lane's row plus its first element 8g.  bf16 rows (hi
// or lo) as they are; f32 values split into the lane's half.
template <bool Coh>
__device__ __forceinline__ void buf_cols_bf16(rsrc_t r, uint32_t off, bool valid, int s,
                                              u32x4 (&rb)[4]) {
    const uint32_t o = off + (uint32_t)s * kKStep * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 v = buf_ld16<Coh>(r, o + 64 * j);
        rb[j] = valid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
}

template <bool Coh>
__device__ __forceinline__ void buf_cols_f32(rsrc_t r, uint32_t off, bool valid, int part, int s,
                                             u32x4 (&rb)[4]) {
    const uint32_t o = off + (uint32_t)s * kKStep * 4;
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_bit_cast(f32x4, buf_ld16<Coh>(r, o + 128 * (j >> 1) + 16 * (j & 1)));
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

// One 16-row bf16 tile: lane (r = l%16, g = l/16) loads row r's elements
// [32j + 8g, 32j + 8g + 8) of step s for MFMA j (A points at element 8g).
__device__ __forceinline__ void load_tile_bf16(const uint16_t *A, int s, u32x4 (&ra)[4]) {
    const uint16_t *p = A + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = ld_weight16(p + 32 * j);
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

// acc[c] += bf16 tile A . columns X[c] for NCG column groups over steps
// [s0, s1): each weight step is loaded once and multiplied against every
// group's columns (one step in flight; NCG = 1 is dense_chunk_x).
template <int NCG>
__device__ __forceinline__ void dense_chunk_xn(const uint16_t *A, const uint16_t *const (&X)[NCG],
                                               const bool (&valid)[NCG], int s0, int s1,
                                               f32x4 (&acc)[NCG]) {
    if constexpr (NCG == 1) {
        dense_chunk_x(A, X[0], valid[0], s0, s1, acc[0]);
    } else {
#pragma unroll 1
        for (int s = s0; s < s1; ++s) {
            u32x4 ra[4], rb[NCG][4];
            load_tile_bf16(A, s, ra);
#pragma unroll
            for (int c = 0; c < NCG; ++c) load_cols_bf16(X[c], valid[c], s, rb[c]);
            fence_schedule();
#pragma unroll
            for (int c = 0; c < NCG; ++c) mfma_tile(ra, rb[c], acc[c]);
        }
    }
}

// Output units: K steps s < Ls run against lat_up and ylat (f32, split into
// hi/lo while loading), the rest against sh_w2 and the shared activation
// (hi/lo bf16 rows).
struct TwoSource {
    const uint16_t *Aa;  // lane's lat_up row + its first element 8g
    const uint16_t *Ab;  // lane's sh_w2 row + 8g
    rsrc_t Ra, Rb;       // ylat, ashhl
    uint32_t Oa, Ob;     // byte offsets of the lane's column row + 8g
    int Ls;              // steps against the first source
};

template <bool Coh>
__device__ __forceinline__ void load_two(const TwoSource &t, bool valid, int part, int s,
                                         u32x4 (&ra)[4], u32x4 (&rb)[4]) {
    if (s < t.Ls) {
        load_tile_bf16(t.Aa, s, ra);
        buf_cols_f32<Coh>(t.Ra, t.Oa, valid, part, s, rb);
    } else {
        load_tile_bf16(t.Ab, s - t.Ls, ra);
        buf_cols_bf16<Coh>(t.Rb, t.Ob, valid, s - t.Ls, rb);
    }
}

template <bool Coh>
__device__ __forceinline__ void dense_chunk_out(const TwoSource &t, bool valid, int part, int s0,
                                                int s1, f32x4 &acc) {
    int s = s0;
#pragma unroll 1
    for (; s + 1 < s1; s += 2) {
        u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
        load_two<Coh>(t, valid, part, s, ra0, rb0);
        load_two<Coh>(t, valid, part, s + 1, ra1, rb1);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
        mfma_tile(ra1, rb1, acc);
    }
    if (s < s1) {
        u32x4 ra0[4], rb0[4];
        load_two<Coh>(t, valid, part, s, ra0, rb0);
        fence_schedule();
        mfma_tile(ra0, rb0, acc);
    }
}

// dense_chunk_out for NCG column groups (per-group byte offsets Oa[c],
// Ob[c]): each weight step is loaded once.  Steps against the f32 source take
// the groups two at a time (their raw loads need twice the registers), the
// bf16 steps all groups at once.
template <bool Coh, int NCG>
__device__ __forceinline__ void dense_chunk_out_n(const TwoSource &t, const uint32_t (&Oa)[NCG],
                                                  const uint32_t (&Ob)[NCG],
                                                  const bool (&valid)[NCG], int part, int s0,
                                                  int s1, f32x4 (&acc)[NCG]) {
#pragma unroll 1
    for (int s = s0; s < s1; ++s) {
        u32x4 ra[4];
        if (s < t.Ls) {
            load_tile_bf16(t.Aa, s, ra);
#pragma unroll
            for (int c0 = 0; c0 < NCG; c0 += 2) {
                constexpr int kPair = NCG > 1 ? 2 : 1;
                u32x4 rb[kPair][4];
#pragma unroll
                for (int q = 0; q < kPair; ++q)
                    if (c0 + q < NCG)
                        buf_cols_f32<Coh>(t.Ra, Oa[c0 + q], valid[c0 + q], part, s, rb[q]);
                fence_schedule();
#pragma unroll
                for (int q = 0; q < kPair; ++q)
                    if (c0 + q < NCG) mfma_tile(ra, rb[q], acc[c0 + q]);
            }
        } else {
            load_tile_bf16(t.Ab, s - t.Ls, ra);
            u32x4 rb[NCG][4];
#pragma unroll
            for (int c = 0; c < NCG; ++c)
                buf_cols_bf16<Coh>(t.Rb, Ob[c], valid[c], s - t.Ls, rb[c]);
            fence_schedule();
#pragma unroll
            for (int c = 0; c < NCG; ++c) mfma_tile(ra, rb[c], acc[c]);
        }
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

// reduce_k1 for NCG accumulators at once (s_red holds NCG slices).
template <int NCG>
__device__ __forceinline__ bool reduce_kn(float *s_red, int wave, int kw, int KW,
                                          f32x4 (&acc)[NCG]) {
    if constexpr (NCG == 1) {
        return reduce_k1(s_red, wave, kw, KW, acc[0]);
    } else {
        const int lane = lane_id();
        constexpr int kSlice = kWG * kWave * 4;
#pragma unroll
        for (int c = 0; c < NCG; ++c) stf4(s_red + c * kSlice + (wave * kWave + lane) * 4, acc[c]);
        __syncthreads();
        if (kw != 0) return false;
        if (KW > 1) {
#pragma unroll
            for (int c = 0; c < NCG; ++c) {
                acc[c] = zero4();
                for (int j = 0; j < KW; ++j)
                    acc[c] += ldf4(s_red + c * kSlice + ((wave + j) * kWave + lane) * 4);
            }
        }
        return true;
    }
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
// Dense-in unit: one tile group of one kind for one column group of tokens.
// ---------------------------------------------------------------------------

enum { KIND_ROUTER = 0, KIND_LATENT = 1, KIND_SHARED = 2 };

// Valid rows of a router tile and of a latent-down tile (a.router_rows,
// a.latent_rows <= 16).  The fused step uses short tiles, which finish the
// router and z early (each unit streams only these rows; MFMA rows past them
// repeat the last row, an L1 hit, and are dropped), so that the routing and
// the expert units that wait for it start sooner; the four-launch step uses
// 16-row tiles (fewer units).

// Tiles: router rows RR t.., latent-down rows RL t.., shared tiles of 8 gate
// rows 8t.. and the 8 matching up rows (so SwiGLU pairs D rows i and 8+i,
// held by lanes l and l+32).  t is the tile index within its kind.  The
// leader wave of a router tile arrives on the router counter; the arrival
// that completes the router sets *s_last (LDS) for its workgroup.  Ends with
// a workgroup barrier.  Coh: the z and shared-activation rows are read by
// other units of the same launch (the fused step).
// Route = false: the routing runs in a later launch; router tiles store their
// scores and keys with plain stores and do not arrive on the counter.
template <bool Coh, bool Route = true>
__device__ __forceinline__ void dense_in_tile(const StepArgs &a, const Role &ro, int kind, int t,
                                              bool active, int cg, float *s_red, int *s_last) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int tt = active ? t : 0;
    const uint16_t *A;
    const int RR = a.router_rows, RL = a.latent_rows;
    if (kind == KIND_ROUTER)
        A = a.router_w + (size_t)(RR * tt + min(n, RR - 1)) * a.H;
    else if (kind == KIND_LATENT)
        A = a.lat_down + (size_t)(RL * tt + min(n, RL - 1)) * a.H;
    else
        A = a.sh_w13 + (size_t)((n < 8 ? 0 : a.Is) + 8 * tt + (n & 7)) * a.H;
    const int b = 16 * cg + n;
    const bool valid = b < a.B;
    const uint16_t *X = a.x + (size_t)(valid ? b : 0) * a.H + 8 * g;
    f32x4 acc = zero4();
    if (active) dense_chunk_x(A + 8 * g, X, valid, ro.kw * a.spc_in, (ro.kw + 1) * a.spc_in, acc);
    const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) {
        if (kind == KIND_ROUTER) {
            const int e = RR * tt + 4 * g;
            if (valid && 4 * g < RR) {
                const f32x4 bv = a.bias ? ldf4(a.bias + e) : zero4();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sv = sigmoidf_(acc[i]);
                    float *ps = a.score + (size_t)b * kMaxExperts + e + i;
                    float *pk = a.key + (size_t)b * kMaxExperts + e + i;
                    if (Route) {
                        store_agent(ps, sv);
                        store_agent(pk, sv + bv[i]);
                    } else {
                        *ps = sv;
                        *pk = sv + bv[i];
                    }
                }
            }
            if (Route && wave_publish(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u &&
                lane == 0)
                *s_last = 1;
        } else if (kind == KIND_LATENT) {
            if (valid && 4 * g < RL) {
                uint16_t *dst = a.zhl + (size_t)b * 2 * a.L + RL * tt + 4 * g;
                store_hl4<Coh>(dst, dst + a.L, acc);
            }
        } else {
            f32x4 up;
#pragma unroll
            for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
            if (valid && g < 2) {
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[i], up[i]);
                uint16_t *dst = a.ashhl + (size_t)b * 2 * a.Is + 8 * tt + 4 * g;
                store_hl4<Coh>(dst, dst + a.Is, v);
            }
        }
    }
    __syncthreads();
}

// Row pointer of lane (row n = lane % 16) in dense-in tile t of `kind`.
__device__ __forceinline__ const uint16_t *dense_in_row(const StepArgs &a, int kind, int tt) {
    const int n = lane_id() & 15;
    const int RR = a.router_rows, RL = a.latent_rows;
    if (kind == KIND_ROUTER) return a.router_w + (size_t)(RR * tt + min(n, RR - 1)) * a.H;
    if (kind == KIND_LATENT) return a.lat_down + (size_t)(RL * tt + min(n, RL - 1)) * a.H;
    return a.sh_w13 + (size_t)((n < 8 ? 0 : a.Is) + 8 * tt + (n & 7)) * a.H;
}

// Epilogue of dense-in tile tt of `kind` for the NCG column groups cg0 ..
// cg0 + NCG - 1 (acc: the tile's full sums, MFMA layout), run by the one
// wave that holds them: router scores and keys (then an arrival on the router
// counter, *s_last set by the arrival that completes it), z or the shared
// activation as hi/lo rows.
template <bool Coh, int NCG, bool Route = true>
__device__ __forceinline__ void dense_in_epilogue(const StepArgs &a, int kind, int tt, int cg0,
                                                  const f32x4 (&acc)[NCG], int *s_last) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int RR = a.router_rows, RL = a.latent_rows;
    if (kind == KIND_ROUTER) {
        const int e = RR * tt + 4 * g;
        // Rows past RR (short router tiles) have no bias entry.
        const f32x4 bv = a.bias && 4 * g < RR ? ldf4(a.bias + e) : zero4();
#pragma unroll
        for (int c = 0; c < NCG; ++c) {
            const int b = 16 * (cg0 + c) + n;
            if (b < a.B && 4 * g < RR) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sv = sigmoidf_(acc[c][i]);
                    float *ps = a.score + (size_t)b * kMaxExperts + e + i;
                    float *pk = a.key + (size_t)b * kMaxExperts + e + i;
                    if (Route) {
                        store_agent(ps, sv);
                        store_agent(pk, sv + bv[i]);
                    } else {
                        *ps = sv;
                        *pk = sv + bv[i];
                    }
                }
            }
        }
        if (Route && wave_publish(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u &&
            lane == 0)
            *s_last = 1;
    } else if (kind == KIND_LATENT) {
#pragma unroll
        for (int c = 0; c < NCG; ++c) {
            const int b = 16 * (cg0 + c) + n;
            if (b < a.B && 4 * g < RL) {
                uint16_t *dst = a.zhl + (size_t)b * 2 * a.L + RL * tt + 4 * g;
                store_hl4<Coh>(dst, dst + a.L, acc[c]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < NCG; ++c) {
            const int b = 16 * (cg0 + c) + n;
            f32x4 up;
#pragma unroll
            for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[c][i], 32);
            if (b < a.B && g < 2) {
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[c][i], up[i]);
                uint16_t *dst = a.ashhl + (size_t)b * 2 * a.Is + 8 * tt + 4 * g;
                store_hl4<Coh>(dst, dst + a.Is, v);
            }
        }
    }
}

// dense_in_tile for the NCG >= 2 column groups cg0 .. cg0 + NCG - 1 (s_red:
// NCG reduction slices): every weight step is loaded once for all of them.
template <bool Coh, int NCG, bool Route = true>
__device__ __forceinline__ void dense_in_tile_n(const StepArgs &a, const Role &ro, int kind, int t,
                                                bool active, int cg0, float *s_red, int *s_last) {
    const int n = lane_id() & 15, g = lane_id() >> 4;
    const int tt = active ? t : 0;
    const uint16_t *A = dense_in_row(a, kind, tt);
    const uint16_t *X[NCG];
    bool valid[NCG];
    f32x4 acc[NCG];
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
        const int b = 16 * (cg0 + c) + n;
        valid[c] = b < a.B;
        X[c] = a.x + (size_t)(valid[c] ? b : 0) * a.H + 8 * g;
        acc[c] = zero4();
    }
    if (active)
        dense_chunk_xn<NCG>(A + 8 * g, X, valid, ro.kw * a.spc_in, (ro.kw + 1) * a.spc_in, acc);
    const bool leader = reduce_kn<NCG>(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) dense_in_epilogue<Coh, NCG, Route>(a, kind, tt, cg0, acc, s_last);
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Expert kernels (2 and 3): shared structure
// ---------------------------------------------------------------------------
//
// A unit is one column unit (one expert, up to 8 of its tokens) and 8 row
// tiles of that expert, one per wave; each wave runs the whole reduction
// length K of its tile, so no partial sums cross waves.  K is taken in chunks
// of S steps (S <= 16, 2048 elements).  Per chunk the workgroup copies the
// unit's activation rows straight from global memory into LDS, every wave
// issues all of its MXFP4 scale and code loads at once (S x 16 B of codes per
// lane), and the MFMAs run step by step as the codes land.  The round trips a
// workgroup waits on are its unit record, the activation copy, then the
// chunk's weights.

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
// lane moves one 16-byte chunk with a direct global -> LDS load (Coh:
// coherent, the rows coming from another unit of the same launch), which
// lands at the block base + 16 * lane.
template <int S, bool Coh, typename RowOf>
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
        if (c < total) __builtin_amdgcn_global_load_lds(g, s_b + 8 * c0, 16, 0, cache_aux<Coh>());
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

// Workgroup barrier after LDS writes that does not wait for global loads in
// flight, as __syncthreads would: each wave's LDS accesses have completed
// (lgkmcnt(0)) when it arrives.
__device__ __forceinline__ void lds_reuse_barrier() {
    fence_schedule();
    // s_waitcnt lgkmcnt(0), with vmcnt and expcnt at their maxima (no wait).
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    fence_schedule();
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
// registers just before their first use.  The wave's S steps are steps
// s_off .. s_off + S - 1 of the staged operand (SS steps per row).
template <int S, int SS = S>
__device__ __forceinline__ void mfma_fp4_chunk(const Fp4Chunk<S> &w, const uint16_t *s_b,
                                               int n_eff, int g, int s_off, f32x4 &acc) {
    const int sh = 8 * g;
    bf16x8 b[2][4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) b[0][jj] = stage_read<SS>(s_b, n_eff, g, s_off, jj);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                b[(s + 1) & 1][jj] = stage_read<SS>(s_b, n_eff, g, s_off + s + 1, jj);
        }
        const float f = e8m0_scale((w.scale[s] >> sh) & 0xFFu);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc = mfma(fp4x8_to_bf16(w.code[s][jj], f), b[s & 1][jj], acc);
    }
}

// ---------------------------------------------------------------------------
// Expert units
// ---------------------------------------------------------------------------

// Reads unit c's record: each lane l < 32 holds word l (its lanes 32..63 a
// copy); returns the expert, pair count and first pair as scalars.  Coh: with
// an agent-scope load (records written by a unit of the same launch).
template <bool Coh>
__device__ __forceinline__ int read_record(const StepArgs &a, int c, int &e, int &nt, int &p0) {
    const int *p = a.cu_rec + (size_t)c * kRecWords + (lane_id() & 31);
    int recw;
    if constexpr (Coh)
        recw = load_agent(p);
    else
        recw = *p;
    e = (int)readlane((uint32_t)recw, R_EXPERT);
    nt = (int)readlane((uint32_t)recw, R_COUNT);
    p0 = (int)readlane((uint32_t)recw, R_PAIR0);
    return recw;
}

// Gate/up unit: column unit c, tile group tg.  Tile t of expert e: gate rows
// 8t .. 8t+7 (MFMA rows 0-7) and up rows I + 8t .. I + 8t + 7 (MFMA rows
// 8-15), so lanes l and l + 32 hold a gate and its up value.  Output: the
// activation of each pair as hi/lo bf16 rows.  `reuse`: s_b may still be read
// by a wave (a barrier comes first).  CohIn: the record and z rows come from
// units of the same launch; CohOut: the activation rows go to units of the
// same launch (agent-scope stores).
template <int S, bool CohIn, bool CohOut, int KS = 1>
__device__ __forceinline__ void w13_unit_rec(const StepArgs &a, int recw, int tg, uint16_t *s_b,
                                             bool &reuse);

template <int S, bool CohIn, bool CohOut>
__device__ __forceinline__ void w13_unit(const StepArgs &a, int c, int tg, uint16_t *s_b,
                                         bool &reuse) {
    int e, nt, p0;
    const int recw = read_record<CohIn>(a, c, e, nt, p0);
    w13_unit_rec<S, CohIn, CohOut>(a, recw, tg, s_b, reuse);
}

// Gate/up unit with its record already read: lane l < 32 holds word l of the
// record (lanes 32..63 a copy).  KS: waves per tile (8 / KS tiles per unit),
// each taking S / KS steps of every chunk; their partial sums meet in LDS and
// are added in wave order before the SwiGLU.
template <int S, bool CohIn, bool CohOut, int KS>
__device__ __forceinline__ void w13_unit_rec(const StepArgs &a, int recw, int tg, uint16_t *s_b,
                                             bool &reuse) {
    static_assert(S % KS == 0 && (KS == 1 || S >= 2), "steps per wave; LDS of the reduction");
    constexpr int SW = S / KS;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4, wave = wave_index();
    const int j = n >> 1, part = n & 1;
    const int OT = a.I >> 3;
    const int nchunk = a.L / (kKStep * S);
    const size_t qrow = a.L / 2, srow = a.L / 32;
    const int t = tg * (kWG / KS) + wave / KS, kh = wave % KS;
    const bool active = t < OT;
    const int e = (int)readlane((uint32_t)recw, R_EXPERT);
    const int nt = (int)readlane((uint32_t)recw, R_COUNT);
    const int p0 = (int)readlane((uint32_t)recw, R_PAIR0);
    const int n_eff = j < nt ? n : part;
    const size_t r = (size_t)e * 2 * a.I + (n < 8 ? 0 : a.I) + 8 * (active ? t : 0) + (n & 7);
    const uint8_t *qp = a.w13_q + r * qrow + 16 * g;
    const uint8_t *sp = a.w13_s + r * srow;
    f32x4 acc = zero4();
    for (int ch = 0; ch < nchunk; ++ch) {
        // Every wave loads and multiplies (a wave past the last tile reads
        // tile 0 again and drops its result), which keeps the load sequence
        // free of branches: the compiler then waits for each step's own loads
        // only.  The staging copies go first, so that the barrier below waits
        // for them alone.
        if (reuse) __syncthreads();  // every wave is done with s_b
        reuse = true;
        Fp4Chunk<SW> w;
        const size_t s0 = (size_t)ch * S + kh * SW;  // the wave's first step
        if constexpr (SW % 4 != 0) load_fp4_scales<SW>(sp + s0 * 4, w);
        fence_schedule();
        stage_operand<S, CohIn>(s_b, a.zhl, a.L, ch * S * kKStep, nt,
                         [&](int jj) { return __shfl(recw, R_TOKEN + jj); });
        fence_schedule();
        if constexpr (SW % 4 == 0) load_fp4_scales<SW>(sp + s0 * 4, w);
        load_fp4_codes<SW>(qp + s0 * 64, w);
        fence_schedule();
        wait_staging<SW>();
        staged_barrier();
        mfma_fp4_chunk<SW, S>(w, s_b, n_eff, g, kh * SW, acc);
    }
    acc = add_pair_column(acc);
    if constexpr (KS > 1) {
        // The tile's KS partial sums, through LDS (the staged operand is no
        // longer read once every wave has passed the barrier).
        float *red = (float *)s_b;
        __syncthreads();
        stf4(red + (size_t)(wave * kWave + lane) * 4, acc);
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int q = 1; q < KS; ++q) {
                const f32x4 o = ldf4(red + (size_t)((wave + q) * kWave + lane) * 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += o[i];
            }
        }
    }
    f32x4 up;
#pragma unroll
    for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32);
    if (kh == 0 && active && j < nt && part == 0 && g < 2) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc[i], up[i]);
        uint16_t *dst = a.acthl + (size_t)(p0 + j) * 2 * a.I + 8 * t + 4 * g;
        store_hl4<CohOut>(dst, dst + a.I, v);
    }
}

// Ordered latent combine, after a down unit's weighted outputs are in pout:
// one arrival per pair of the unit on its token's counter for tile group tg
// (k arrivals complete a token's group); the unit that completes a token
// sums the token's k rows of pout over the group's latent rows [r0, r0 +
// rows) in pair order, j = 0 .. k - 1 (ascending expert id), writes them to
// ylat and clears the counter.  The sums therefore do not depend on the
// order in which units run.  Starts after every wave's pout stores have
// completed and a workgroup barrier; ends with a workgroup barrier.
__device__ __forceinline__ void ordered_combine(const StepArgs &a, int recw, int nt, int tg,
                                                int r0, int rows, int *s_done) {
    const int lane = lane_id(), k = a.k;
    if (wave_index() == 0) {
        const int tok = __shfl(recw, R_TOKEN + (lane < nt ? lane : 0));
        uint32_t *ctr = a.cctr + ((size_t)tok * kOrdGroups + tg) * kOrdStride;
        uint32_t old = 0u;
        if (lane < nt) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane < 8) s_done[lane] = lane < nt && old == (uint32_t)k - 1u ? tok : -1;
        if (lane < nt && old == (uint32_t)k - 1u) store_agent(ctr, 0u);  // for the next step
    }
    __syncthreads();
    const rsrc_t rp = buf_rsrc(a.pout);
    const int q4 = rows / 4;  // 16-byte column chunks of one token
    for (int it = threadIdx.x; it < 8 * q4; it += kWGThreads) {
        const int b = s_done[it / q4];
        if (b < 0) continue;
        const int r = r0 + 4 * (it % q4);
        f32x4 sum = zero4();
        for (int j0 = 0; j0 < k; j0 += 16) {
            u32x4 v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q)
                v[q] = buf_ld16<true>(rp, (uint32_t)((((size_t)b * k + min(j0 + q, k - 1)) * a.L + r) * 4));
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (j0 + q < k) sum += __builtin_bit_cast(f32x4, v[q]);
        }
        stf4(a.ylat + (size_t)b * a.L + r, sum);
    }
    __syncthreads();
}

// Down unit: column unit c, tile group tg.  Tile t of expert e: latent rows
// 16t .. 16t+15; the routing weight of each pair scales its column before the
// f32 atomic add into ylat.  Coh: the record and activation rows come from
// units of the same launch.  KS: waves per tile (8 / KS tiles per unit), each
// taking S / KS steps of every chunk; the KS partial sums are added through
// LDS, in wave order.  Ord: the weighted outputs go to pout instead and
// ordered_combine forms ylat.
template <int S, bool Coh, int KS = 1, bool Ord = false>
__device__ __forceinline__ void w2_unit(const StepArgs &a, int c, int tg, uint16_t *s_b,
                                        bool &reuse) {
    static_assert(S % KS == 0, "steps per wave");
    constexpr int SW = S / KS;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4, wave = wave_index();
    const int j = n >> 1, part = n & 1;
    const int OT = a.L >> 4;
    const int nchunk = a.I / (kKStep * S);
    const size_t qrow = a.I / 2, srow = a.I / 32;
    const int t = tg * (kWG / KS) + wave / KS, kh = wave % KS;
    const bool active = t < OT;
    int e, nt, p0;
    const int recw = read_record<Coh>(a, c, e, nt, p0);
    const int jc = j < nt ? j : 0;
    const int tok_j = __shfl(recw, R_TOKEN + jc);
    const float w_j = __int_as_float(__shfl(recw, R_WEIGHT + jc));
    const int n_eff = j < nt ? n : part;
    const size_t r = (size_t)e * a.L + 16 * (active ? t : 0) + n;
    const uint8_t *qp = a.w2_q + r * qrow + 16 * g;
    const uint8_t *sp = a.w2_s + r * srow;
    f32x4 acc = zero4();
    for (int ch = 0; ch < nchunk; ++ch) {
        // As in w13_unit.
        if (reuse) __syncthreads();
        reuse = true;
        Fp4Chunk<SW> w;
        const size_t s0 = (size_t)ch * S + kh * SW;  // the wave's first step
        if constexpr (SW % 4 != 0) load_fp4_scales<SW>(sp + s0 * 4, w);
        fence_schedule();
        stage_operand<S, Coh>(s_b, a.acthl, a.I, ch * S * kKStep, nt,
                         [&](int jj) { return p0 + jj; });
        fence_schedule();
        if constexpr (SW % 4 == 0) load_fp4_scales<SW>(sp + s0 * 4, w);
        load_fp4_codes<SW>(qp + s0 * 64, w);
        fence_schedule();
        wait_staging<SW>();
        staged_barrier();
        mfma_fp4_chunk<SW, S>(w, s_b, n_eff, g, kh * SW, acc);
    }
    acc = add_pair_column(acc);
    if constexpr (!Ord) {
        // The unit's weighted sums meet in LDS as [KS][token][row] (rows of
        // its 8 / KS tiles, the staged operand no longer read once every wave
        // has passed the barrier); then each wave adds 64 consecutive rows of
        // one token per atomic instruction, the KS partial sums added first.
        constexpr int RW = 16 * (kWG / KS);  // latent rows of the unit
        float *red = (float *)s_b;
        static_assert(KS * 8 * RW * 4 <= 8 * Stage<1>::kChunks * 2, "reduction buffer");
        __syncthreads();
        if (active && j < nt && part == 0) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = w_j * acc[i];
            stf4(red + (size_t)(kh * 8 + j) * RW + 16 * (wave / KS) + 4 * g, v);
        }
        __syncthreads();
        const int r0 = 16 * tg * (kWG / KS);
        const int rows = min(RW, a.L - r0);
        for (int it = threadIdx.x; it < nt * RW; it += kWGThreads) {
            const int jj = it / RW, rr = it % RW;
            const int tok = __shfl(recw, R_TOKEN + jj);
            if (rr < rows) {
                float v = red[(size_t)jj * RW + rr];
#pragma unroll
                for (int q = 1; q < KS; ++q) v += red[(size_t)(q * 8 + jj) * RW + rr];
                unsafeAtomicAdd(a.ylat + (size_t)tok * a.L + r0 + rr, v);
            }
        }
    } else {
        if constexpr (KS > 1) {
            float *red = (float *)s_b;
            __syncthreads();  // every wave is done with the staged operand
            stf4(red + (size_t)(wave * kWave + lane) * 4, acc);
            __syncthreads();
            if (kh == 0) {
#pragma unroll
                for (int q = 1; q < KS; ++q) acc += ldf4(red + (size_t)((wave + q) * kWave + lane) * 4);
            }
        }
        // The pair's place in token order: b k + (its expert's rank among the
        // token's experts).
        const int pj = a.pair_slot[p0 + jc];
        if (kh == 0 && active && j < nt && part == 0) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = w_j * acc[i];
            buf_st16<true>(buf_rsrc(a.pout), (uint32_t)((((size_t)pj * a.L) + 16 * t + 4 * g) * 4),
                           __builtin_bit_cast(u32x4, v));
        }
        wait_vm_all();    // this wave's pout stores have completed
        __syncthreads();  // ... and every wave's; s_b is free
        const int r0 = 16 * (kWG / KS) * tg;
        ordered_combine(a, recw, nt, tg, r0, min(16 * (kWG / KS), a.L - r0), (int *)s_b);
    }
}

// ---------------------------------------------------------------------------
// Output unit: one tile of RT = out_rows <= 16 rows (MFMA rows past RT repeat
// the tile's last row and are dropped) for one column group of 8 tokens.
// ---------------------------------------------------------------------------

enum { OUT_BOTH = 0, OUT_SHARED = 1, OUT_LATENT = 2 };

// OUT_BOTH: latent-up and shared-down in one pass, one bf16 rounding (the
// four-launch step).  OUT_SHARED: shared-down only, f32 sums to ysh.
// OUT_LATENT: latent-up, plus ysh, one bf16 rounding.  K steps: the wave's
// slice [kw * spc, (kw + 1) * spc).  Ends with a workgroup barrier.  Coh:
// ylat and the shared activation come from units of the same launch.
template <bool Coh>
__device__ __forceinline__ void out_tile(const StepArgs &a, const Role &ro, int mode, int t,
                                         bool active, int cg, int spc, float *s_red);

// OUT_BOTH for the NCG column groups cg0 .. cg0 + NCG - 1 (s_red: NCG
// reduction slices); every weight step is loaded once for all of them.
template <int NCG>
__device__ __forceinline__ void out_tile_n(const StepArgs &a, const Role &ro, int t, bool active,
                                           int cg0, float *s_red) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int RT = a.out_rows;
    const int h0 = RT * (active ? t : 0);
    const size_t h = min(h0 + min(n, RT - 1), a.H - 1);
    TwoSource ts;
    ts.Aa = a.lat_up + h * a.L + 8 * g;
    ts.Ab = a.sh_w2 + h * a.Is + 8 * g;
    ts.Ra = buf_rsrc(a.ylat);
    ts.Rb = buf_rsrc(a.ashhl);
    ts.Ls = a.L / kKStep;
    uint32_t Oa[NCG], Ob[NCG];
    bool valid[NCG];
    f32x4 acc[NCG];
#pragma unroll
    for (int c = 0; c < NCG; ++c) {
        const int b = 8 * (cg0 + c) + col;
        valid[c] = b < a.B;
        const int bb = valid[c] ? b : 0;
        Oa[c] = (uint32_t)(((size_t)bb * a.L + 8 * g) * 4);
        Ob[c] = (uint32_t)((((size_t)bb * 2 + part) * a.Is + 8 * g) * 2);
        acc[c] = zero4();
    }
    if (active) {
        if constexpr (NCG == 1) {  // one group: two steps in flight
            ts.Oa = Oa[0];
            ts.Ob = Ob[0];
            dense_chunk_out<false>(ts, valid[0], part, ro.kw * a.spc_out, (ro.kw + 1) * a.spc_out,
                                   acc[0]);
        } else {
            dense_chunk_out_n<false, NCG>(ts, Oa, Ob, valid, part, ro.kw * a.spc_out,
                                          (ro.kw + 1) * a.spc_out, acc);
        }
    }
    const bool leader = reduce_kn<NCG>(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) {
#pragma unroll
        for (int c = 0; c < NCG; ++c) {
            const f32x4 v = add_pair_column(acc[c]);
            const int b = 8 * (cg0 + c) + col;
            if (valid[c] && part == 0) {
                const size_t o = (size_t)b * a.H + h0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * g + i;
                    if (r < RT && h0 + r < a.H) a.out[o + r] = (uint16_t)bf16_rne(v[i]);
                }
            }
        }
    }
    __syncthreads();
}

template <bool Coh>
__device__ __forceinline__ void out_tile(const StepArgs &a, const Role &ro, int mode, int t,
                                         bool active, int cg, int spc, float *s_red) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int RT = a.out_rows;
    const int b = 8 * cg + col;
    const bool valid = b < a.B;
    const int bb = valid ? b : 0;
    const int h0 = RT * (active ? t : 0);
    const size_t h = min(h0 + min(n, RT - 1), a.H - 1);
    TwoSource ts;
    ts.Aa = a.lat_up + h * a.L + 8 * g;
    ts.Ab = a.sh_w2 + h * a.Is + 8 * g;
    ts.Ra = buf_rsrc(a.ylat);
    ts.Rb = buf_rsrc(a.ashhl);
    ts.Oa = (uint32_t)(((size_t)bb * a.L + 8 * g) * 4);
    ts.Ob = (uint32_t)((((size_t)bb * 2 + part) * a.Is + 8 * g) * 2);
    ts.Ls = mode == OUT_SHARED ? 0 : a.L / kKStep;
    f32x4 acc = zero4();
    if (active) dense_chunk_out<Coh>(ts, valid, part, ro.kw * spc, (ro.kw + 1) * spc, acc);
    const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) {
        acc = add_pair_column(acc);
        if (valid && part == 0) {
            const size_t o = (size_t)b * a.H + h0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                if (r < RT && h0 + r < a.H) {
                    if (mode == OUT_SHARED) {
                        store_agent(a.ysh + o + r, acc[i]);
                    } else {
                        const float v = mode == OUT_LATENT ? acc[i] + load_agent(a.ysh + o + r) : acc[i];
                        a.out[o + r] = (uint16_t)bf16_rne(v);
                    }
                }
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Completion counters shared by workgroups of one launch
// ---------------------------------------------------------------------------

constexpr uint32_t kSpinLimit = 1u << 15;  // ~50 ms of polls: far beyond any legitimate wait

// Counter increment after the whole workgroup's stores have completed.
__device__ __forceinline__ void wg_publish(uint32_t *ctr, uint32_t v = 1u) {
    wait_vm_all();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns once *ctr >= target (the whole workgroup waits at the barrier).
__device__ __forceinline__ void wg_wait(const StepArgs &a, const uint32_t *ctr, uint32_t target) {
    if (threadIdx.x == 0) {
        uint32_t polls = 0;
        while (load_agent(ctr) < target) {
            if (++polls >= kSpinLimit) {
                __hip_atomic_fetch_or(&a.gctr[G_ERROR], 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(32);
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Four-launch step
// ---------------------------------------------------------------------------

// Kernel 0 (f32 router only): logits, scores and keys with plain f32 FMAs;
// the workgroup whose arrival completes the router routes the step.
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
    if (s_last) route_step<false>(route_args(a), &s_route, kWavesPerBlock);
}

// The last routing unit of a launch: every unit's selections into LDS
// (16-byte coherent loads, all issued before the first use: one round trip;
// the arrays are 256-byte aligned in the workspace, so the last chunk's bytes
// past B k are inside it and unused), then the metadata.
__device__ __forceinline__ void routed_meta(const StepArgs &a, const RouteArgs &ra, RouteLds &s_route) {
    static_assert(kMaxBatch * kMaxTopK <= 2 * 4 * kWGThreads, "two chunks per thread");
    const int P = a.B * a.k, nc = (P + 3) >> 2;
    const rsrc_t ri = buf_rsrc(a.idx), rw = buf_rsrc(a.wsel);
    u32x4 vi[2], vw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = min((int)threadIdx.x + kWGThreads * h, nc - 1);
        vi[h] = buf_ld16<true>(ri, (uint32_t)c * 16);
        vw[h] = buf_ld16<true>(rw, (uint32_t)c * 16);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = (int)threadIdx.x + kWGThreads * h;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (4 * c + q < P) {
                s_route.idx[4 * c + q] = (int16_t)vi[h][q];
                s_route.w[4 * c + q] = __uint_as_float(vw[h][q]);
            }
    }
    __syncthreads();
    build_meta<false, false>(ra, s_route, kWG);  // read by later launches only
    if (threadIdx.x == 0) store_agent(&a.gctr[G_ROUTED], 0u);  // ready for the next step
}

// Routing units (large batches), after the `units` dense units of the
// launch: unit r routes tokens 8r .. 8r + 7 (a wave each) once the router is
// complete, and the last routing unit to finish builds the metadata from
// every unit's selections.  A routing unit waits only for router units,
// which come first in the grid.
__device__ __forceinline__ void routing_units(const StepArgs &a, int units, RouteLds &s_route,
                                              int *s_flag) {
    for (int r = (int)blockIdx.x - units; r >= 0 && r < a.route_units; r += gridDim.x) {
        wg_wait(a, &a.gctr[G_ROUTER_DONE], (uint32_t)a.router_target);
        const RouteArgs ra = route_args(a);
        const int b = kWG * r + wave_index();
        if (b < a.B) topk_token<true>(ra, b, s_route);
        wait_vm_all();
        __syncthreads();
        if (threadIdx.x == 0)
            *s_flag = __hip_atomic_fetch_add(&a.gctr[G_ROUTED], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)a.route_units - 1u;
        __syncthreads();
        if (*s_flag) routed_meta(a, ra, s_route);
    }
}

// Routing units of the large-batch dense-in launch when it holds the bf16
// router (its router row groups store K-slice partial sums and never add
// them): unit r routes tokens kRouteTokensTp r, ... once every router slice
// has arrived.  Thread i takes token i / (E / 4) and experts 4q .. 4q + 3
// (q = i % (E / 4)): it adds that token's router partials of those experts
// over the slices in slice order (the router slices store them token-major
// for this, so a wave's loads are contiguous) and keeps scores and keys in
// LDS (kv: the x staging area, unused by routing units).  Waves 0 .. kRouteTokensTp - 1 then select one token's
// experts each, the last unit to finish builds the metadata, and the scores
// and keys go to global memory last.  One round trip for the partials
// instead of a chain of slice sums, router epilogues and key loads.
__device__ __forceinline__ void routing_units_tp(const StepArgs &a, int units, RouteLds &s_route,
                                                 float *kv, int *s_flag) {
    static_assert(sizeof(s_route.cand_key) / sizeof(s_route.cand_key[0]) >= kRouteTokensTp,
                  "a candidate row per selecting wave");
    const int nsteps = a.H / kKStep, nsl = (nsteps + a.kx_sps_r - 1) / a.kx_sps_r;
    const int per = a.E / 4;  // 16-byte chunks of a token's router row
    const rsrc_t rrpart = buf_rsrc(a.rpart);
    for (int r = (int)blockIdx.x - units; r >= 0 && r < a.route_units; r += gridDim.x) {
        wg_wait(a, &a.gctr[G_ROUTER_DONE], (uint32_t)a.router_target);
        const int i = threadIdx.x, j = i / per, q = i % per;
        const int b = kRouteTokensTp * r + j;
        if (j < kRouteTokensTp && b < a.B) {
            u32x4 v[kMaxSlices];
#pragma unroll
            for (int k = 0; k < kMaxSlices; ++k) {
                const int kk = min(k, nsl - 1);
                v[k] = buf_ld16<true>(rrpart, (uint32_t)((((size_t)kk * a.B + b) * kMaxExperts + 4 * q) * 4));
            }
            f32x4 sum = zero4();
#pragma unroll
            for (int k = 0; k < kMaxSlices; ++k)
                if (k < nsl) sum += __builtin_bit_cast(f32x4, v[k]);
            const int e = 4 * q;
            const f32x4 bv = a.bias ? ldf4(a.bias + e) : zero4();
            float *kr = kv + (size_t)j * 2 * kMaxExperts;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float sv = sigmoidf_(sum[q]);
                kr[e + q] = sv + bv[q];
                kr[kMaxExperts + e + q] = sv;
            }
        }
        __syncthreads();
        // Wave j selects token kRouteTokensTp r + j (threshold selection, its
        // own candidate row).
        const RouteArgs ra = route_args(a);
        const int jw = wave_index(), bb = kRouteTokensTp * r + jw;
        if (jw < kRouteTokensTp && bb < a.B) {
            const float *kr = kv + (size_t)jw * 2 * kMaxExperts;
            topk_token<true, true>(ra, bb, s_route, true, kr, kr + kMaxExperts);
        }
        wait_vm_all();
        __syncthreads();
        if (threadIdx.x == 0)
            *s_flag = __hip_atomic_fetch_add(&a.gctr[G_ROUTED], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)a.route_units - 1u;
        __syncthreads();
        if (*s_flag) routed_meta(a, ra, s_route);
        // The units' scores and keys for later launches and the caller, from
        // LDS with 16-byte stores once the selections are published: off
        // the routing's chain of round trips.
        const int q4n = a.E / 4;
        for (int x = threadIdx.x; x < kRouteTokensTp * q4n; x += kWGThreads) {
            const int jj = x / q4n, e4 = 4 * (x % q4n), bq = kRouteTokensTp * r + jj;
            if (bq < a.B) {
                const float *kr = kv + (size_t)jj * 2 * kMaxExperts;
                stf4(a.key + (size_t)bq * kMaxExperts + e4, *(const f32x4 *)(kr + e4));
                stf4(a.score + (size_t)bq * kMaxExperts + e4, *(const f32x4 *)(kr + kMaxExperts + e4));
            }
        }
        __syncthreads();  // kv is read before a next unit of this workgroup writes it
    }
}

// Prefetch units, after the routing units: unit r reads bytes [r U, r U + U)
// (U = kPfUnit) of a following layer's router and latent-down rows with
// plain loads, once the router is complete, so that those rows sit in the
// last-level cache when that layer's step streams them; the values are
// dropped.  They run while the routing leaves the memory idle.
constexpr int kPfUnit = 256 * 1024;
__device__ __forceinline__ void prefetch_units(const StepArgs &a, int first) {
    const int r = (int)blockIdx.x - first;
    if (r < 0 || r >= a.pf_units) return;
    wg_wait(a, &a.gctr[G_ROUTER_DONE], (uint32_t)a.router_target);
    constexpr int kPer = kPfUnit / (kWGThreads * 16);  // 16-byte loads per thread
    constexpr int kBatch = 8;
    const uint64_t total = a.pf_bytes0 + a.pf_bytes1;
    uint32_t acc = 0;
    for (int i0 = 0; i0 < kPer; i0 += kBatch) {
        u32x4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            uint64_t off = (uint64_t)r * kPfUnit + ((uint64_t)(i0 + j) * kWGThreads + threadIdx.x) * 16;
            off = off < total ? off : 0;  // past the end: re-read the first chunk
            const uint8_t *p = off < a.pf_bytes0 ? a.pf0 + off : a.pf1 + (off - a.pf_bytes0);
            v[j] = ld16(p);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    if (a.pf_units < 0) a.out[acc & 1] = 0;  // never taken (pf_units > 0 here): keeps the loads
}

// Kernel 1: dense-in units over tiles [dense_lo, dense_hi) of the list
// [router | latent | shared]; each unit covers all NCG = ceil(B / 16) column
// groups, so every weight tile is read once per step.
// The routing image of a dense-in launch that routes (none otherwise).
template <bool Route>
struct RouteShared {
    RouteLds s;
};
template <>
struct RouteShared<false> {};

// Route = false: the routing runs at the start of the gate/up launch (at most
// 8 tokens), so this launch holds no routing code and only streams weights.
template <int NCG, bool Route>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_dense_in(const StepArgs a) {
    __shared__ RouteShared<Route> s_rs;
    __shared__ float s_red[NCG * kWG * kWave * 4];
    __shared__ int s_last;
    const Role ro = role_of(a.kw_in);
    if (threadIdx.x == 0) s_last = 0;
    // The latent combine accumulates into ylat with atomics later in the step.
    if (a.zero_ylat)
        for (int i = (blockIdx.x * kWGThreads + threadIdx.x) * 4; i < a.B * a.L;
             i += gridDim.x * kWGThreads * 4)
            stf4(a.ylat + i, zero4());
    const int n_rt = a.n_rtiles, n_lt = a.L / a.latent_rows;
    const int ncg = NCG == 1 ? (a.B + 15) >> 4 : 1;  // 1 whenever B <= 16
    const int units = dense_units(a.dense_hi - a.dense_lo, ro.RW, ncg);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int cg, tg;
        dense_unit(u, ncg, cg, tg);
        const int t = a.dense_lo + tg * ro.RW + ro.rg;
        const bool active = t < a.dense_hi;
        const int kind = t < n_rt ? KIND_ROUTER : t < n_rt + n_lt ? KIND_LATENT : KIND_SHARED;
        const int tl = kind == KIND_ROUTER ? t : kind == KIND_LATENT ? t - n_rt : t - n_rt - n_lt;
        if constexpr (NCG == 1)
            dense_in_tile<false, Route>(a, ro, kind, tl, active, cg, s_red, &s_last);
        else
            dense_in_tile_n<false, NCG, Route>(a, ro, kind, tl, active, 0, s_red, &s_last);
        if constexpr (Route) {
            if (s_last && !a.route_units) {  // this workgroup completed the router: route the step
                route_step<false>(route_args(a), &s_rs.s, kWG);
                __syncthreads();
                if (threadIdx.x == 0) s_last = 0;
            }
        }
    }
    if constexpr (Route) {
        routing_units(a, units, s_rs.s, &s_last);
        prefetch_units(a, units + a.route_units);
    }
}

// Kernel 1 up to 2 tokens: the tokens' x rows are staged in LDS by every
// workgroup, so a wave's registers hold weights only and six of its K steps
// stay in flight (a ring of six step buffers, each refilled with the step six
// ahead as soon as its MFMAs have read it); a wave's chain of round
// trips, not the bandwidth, sets the launch's time at these batches.  The
// staging loads go out first, the six first weight steps behind them, and
// only the staging loads are waited for before the LDS copy (vector loads
// complete in issue order).  One unit per workgroup (no loop, so that no wait
// carries over a loop edge); tiles, K split and epilogues as in k_dense_in.
// Route: as in k_dense_in, the workgroup whose router arrival completes the
// router then routes the step, in LDS that x no longer needs; prefetch units
// follow the dense units.
constexpr int kXlTokens = 2;
// 3 to 8 tokens: the same kernel with all 8 rows staged (131 KB of LDS, one
// workgroup per compute unit, whose waves may hold twice the registers: the
// staged x and the weight ring together).  Instead of two weight steps in
// flight per wave with the columns loaded from memory by every wave.
constexpr int kXlTokensWide = 8;
constexpr int kXlRing = 4;       // weight steps in flight per wave (output kernel); the least spc
constexpr int kXlDenseRing = 6;  // ... dense-in (K3 batch 1: 29.4 -> 28.5 us against 4)
constexpr int kXlPad = 8;  // elements after each staged row: the rows' equal columns on distinct banks
template <bool Route, int NT>
union XlShared {
    uint16_t x[NT * (kMaxDenseK + kXlPad)];
    RouteLds route;
};
template <int NT>
union XlShared<false, NT> {
    uint16_t x[NT * (kMaxDenseK + kXlPad)];
};

// The dense-in tile of the workgroup with NT token rows of x staged in LDS.
template <bool Route, int NT>
__device__ __forceinline__ void dense_in_xl_body(const StepArgs &a, XlShared<Route, NT> &s_u,
                                                 float *s_red, int &s_last) {
    uint16_t *s_x = s_u.x;
    const Role ro = role_of(a.kw_in);
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    if (threadIdx.x == 0) s_last = 0;
    if (a.zero_ylat)
        for (int i = (blockIdx.x * kWGThreads + threadIdx.x) * 4; i < a.B * a.L;
             i += gridDim.x * kWGThreads * 4)
            stf4(a.ylat + i, zero4());
    const int units = dense_units(a.dense_hi - a.dense_lo, ro.RW, 1);
    if ((int)blockIdx.x >= units) {
        if constexpr (Route) prefetch_units(a, units + a.route_units);
        return;
    }
    int cg, tg;
    dense_unit(blockIdx.x, 1, cg, tg);
    const int n_rt = a.n_rtiles, n_lt = a.L / a.latent_rows;
    const int t0 = a.dense_lo + tg * ro.RW + ro.rg;
    const bool active = t0 < a.dense_hi;
    const int kind = t0 < n_rt ? KIND_ROUTER : t0 < n_rt + n_lt ? KIND_LATENT : KIND_SHARED;
    const int tl = kind == KIND_ROUTER ? t0 : kind == KIND_LATENT ? t0 - n_rt : t0 - n_rt - n_lt;
    const int tt = active ? tl : 0;
    const uint16_t *A = dense_in_row(a, kind, tt) + 8 * g;
    const int ns = a.spc_in, s0 = ro.kw * ns;  // kXlRing <= ns <= kMaxStepsPerChunk (host)
    // x chunks of this thread (16 bytes each): c = threadIdx.x + kWGThreads q.
    constexpr int kQx = NT * kMaxDenseK / 8 / kWGThreads;
    const int nq = a.B * a.H / 8;
    u32x4 xs[kQx];
#pragma unroll
    for (int q = 0; q < kQx; ++q) xs[q] = ld16(a.x + 8 * (size_t)min((int)threadIdx.x + kWGThreads * q, nq - 1));
    fence_schedule();
    u32x4 w[kXlDenseRing][4];
#pragma unroll
    for (int i = 0; i < kXlDenseRing; ++i) load_tile_bf16(A, min(s0 + i, s0 + ns - 1), w[i]);
    fence_schedule();
    // vmcnt(24): the x loads have landed (vmcnt in bits [3:0] and [15:14]).
    constexpr int kWl = 4 * kXlDenseRing;
    __builtin_amdgcn_s_waitcnt((kWl & 15) | ((kWl >> 4) << 14) | 0x0F70);
    const int rq = a.H / 8, xst = a.H + kXlPad;  // chunks per token row; staged row stride
#pragma unroll
    for (int q = 0; q < kQx; ++q) {
        const int c = (int)threadIdx.x + kWGThreads * q;
        if (c < nq) *(u32x4 *)(s_x + (size_t)(c / rq) * xst + 8 * (c % rq)) = xs[q];
    }
    lds_reuse_barrier();  // x is in LDS for every wave (weight loads still in flight)
    const uint16_t *xr = s_x + (size_t)(n < a.B ? n : 0) * xst + 8 * g;
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < kMaxStepsPerChunk; ++i) {
        if (i < ns) {
            const uint16_t *xp = xr + (size_t)(s0 + i) * kKStep;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = mfma(as_bf16x8(w[i % kXlDenseRing][j]), as_bf16x8(*(const u32x4 *)(xp + 32 * j)), acc);
            if (i + kXlDenseRing < ns) load_tile_bf16(A, s0 + i + kXlDenseRing, w[i % kXlDenseRing]);
        }
    }
    const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) {
        f32x4 sum[1] = {acc};
        dense_in_epilogue<false, 1, Route>(a, kind, tt, 0, sum, &s_last);
    }
    if constexpr (Route) {
        __syncthreads();  // s_last is set; every wave is done with x
        if (s_last) route_step<false>(route_args(a), &s_u.route, kWG);
    }
}

template <bool Route>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_dense_in_xl(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) XlShared<Route, kXlTokens> s_u;
    __shared__ float s_red[kWG * kWave * 4];
    __shared__ int s_last;
    dense_in_xl_body<Route, kXlTokens>(a, s_u, s_red, s_last);
}

template <bool Route>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(2)))
k_dense_in_xl8(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) XlShared<Route, kXlTokensWide> s_u;
    __shared__ float s_red[kWG * kWave * 4];
    __shared__ int s_last;
    dense_in_xl_body<Route, kXlTokensWide>(a, s_u, s_red, s_last);
}

// Sum over the nsl slices of tile t's partials part[k][t][c][lane] (T tiles
// per slice), in slice order.  The loads of a batch of slices are all issued
// before their sums (indices clamped to the last slice, the extra values
// dropped), so a batch costs one round trip.
template <int NCG>
__device__ __forceinline__ void sum_slices(rsrc_t rpart, int nsl, int T, int t, f32x4 (&sum)[NCG]) {
    constexpr int SB = NCG <= 4 ? 16 / NCG : 2;  // slices per batch: 16 loads
    const int lane = lane_id();
#pragma unroll
    for (int c = 0; c < NCG; ++c) sum[c] = zero4();
    for (int k0 = 0; k0 < nsl; k0 += SB) {
        f32x4 v[SB][NCG];
#pragma unroll
        for (int q = 0; q < SB; ++q) {
            const int k = min(k0 + q, nsl - 1);
#pragma unroll
            for (int c = 0; c < NCG; ++c)
                v[q][c] = __builtin_bit_cast(
                    f32x4, buf_ld16<true>(rpart, (uint32_t)(((((size_t)k * T + t) * NCG + c) * kWave + lane) * 16)));
        }
#pragma unroll
        for (int q = 0; q < SB; ++q)
            if (k0 + q < nsl) {
#pragma unroll
                for (int c = 0; c < NCG; ++c) sum[c] += v[q][c];
            }
    }
}

// Kernel 1 for more than 16 tokens (NCG = ceil(B / 16) >= 2 column groups).
// A unit is a row group (8 tiles, one per wave) times a K slice of a.kx_sps
// steps.  Per pair of steps the workgroup copies the x columns of every
// token (64 rows x 128 bf16 per step) straight into LDS once, and all 8 waves
// multiply their own weight rows against that copy: x is read once per row
// group and step instead of once per tile and step.  A slice's partial sums
// go to a.part; the last slice of a row group to arrive sums them in slice
// order and runs the tile epilogues, so the results do not depend on the
// order of arrival.  The router's row groups come first, in slices of
// a.kx_sps_r steps: shorter units, done early in the launch.  Their slices
// only store partial sums and arrive on the router counter; the routing
// units (routing_units_tp) add each token's router partials themselves, so
// that the routing runs while the other row groups still stream their
// weights.
constexpr int kXRows = 64;  // token rows of one staged step

// Copies the x columns of step s into buf: row b (token b; rows past B copy
// token 0 and are never used) at b * 128 elements, its 16-byte chunk q at
// position q ^ (b & 15), so that the 16 rows of one MFMA operand read sit on
// distinct banks.  Two 16-byte copies per thread, landing at their wave's
// block base + 16 * lane.
__device__ __forceinline__ void stage_x_step(uint16_t *buf, const StepArgs &a, int s) {
    const int lane = lane_id(), wave = wave_index();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c0 = 64 * (wave + kWG * h), c = c0 + lane;
        const int b = c >> 4, q = (c & 15) ^ (b & 15);
        const uint16_t *gp = a.x + (size_t)(b < a.B ? b : 0) * a.H + (size_t)s * kKStep + 8 * q;
        __builtin_amdgcn_global_load_lds(gp, buf + 8 * c0, 16, 0, 0);
    }
}

// MFMA j's x operand of column group c from a staged step: token 16c + n,
// elements [32j + 8g, 32j + 8g + 8).
__device__ __forceinline__ bf16x8 x_operand(const uint16_t *buf, int c, int j) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    return as_bf16x8(*(const u32x4 *)(buf + (16 * c + n) * kKStep + 8 * ((4 * j + g) ^ n)));
}

template <int NCG>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_dense_in_kx(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kXRows * kKStep];
    static_assert(sizeof(s_x) >= kRouteTokensTp * 2 * kMaxExperts * sizeof(float),
                  "routing units keep their tokens' keys and scores in the x staging area");
    __shared__ RouteLds s_route;
    __shared__ int s_last, s_arrive;
    const int lane = lane_id(), wave = wave_index(), g = lane >> 4;
    if (threadIdx.x == 0) s_last = 0;
    if (a.zero_ylat)
        for (int i = (blockIdx.x * kWGThreads + threadIdx.x) * 4; i < a.B * a.L;
             i += gridDim.x * kWGThreads * 4)
            stf4(a.ylat + i, zero4());
    const int n_rt = a.n_rtiles, n_lt = a.L / a.latent_rows;
    const int nsteps = a.H / kKStep;
    const int nsl_r = (nsteps + a.kx_sps_r - 1) / a.kx_sps_r, nsl_o = (nsteps + a.kx_sps - 1) / a.kx_sps;
    const int nrg = (a.dense_hi - a.dense_lo + kWG - 1) / kWG;
    const int units_r = a.kx_rg_r * nsl_r, units = units_r + (nrg - a.kx_rg_r) * nsl_o;
    const rsrc_t rpart = buf_rsrc(a.part), rrpart = buf_rsrc(a.rpart);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const bool short_sl = u < units_r;
        const int nsl = short_sl ? nsl_r : nsl_o, sps = short_sl ? a.kx_sps_r : a.kx_sps;
        const int v = short_sl ? u : u - units_r;
        const int rg = (short_sl ? 0 : a.kx_rg_r) + v / nsl, ks = v % nsl;
        const int t = a.dense_lo + rg * kWG + wave;
        const bool active = t < a.dense_hi;
        const int kind = t < n_rt ? KIND_ROUTER : t < n_rt + n_lt ? KIND_LATENT : KIND_SHARED;
        const int tl = kind == KIND_ROUTER ? t : kind == KIND_LATENT ? t - n_rt : t - n_rt - n_lt;
        const int tt = active ? tl : 0;
        const uint16_t *A = dense_in_row(a, kind, tt) + 8 * g;
        const int s0 = ks * sps, s1 = min(nsteps, s0 + sps);
        f32x4 acc[NCG];
#pragma unroll
        for (int c = 0; c < NCG; ++c) acc[c] = zero4();
        for (int s = s0; s < s1; s += 2) {
            const bool two = s + 1 < s1;
            __syncthreads();  // every wave is done with the staged copies
            u32x4 ra0[4], ra1[4];
            stage_x_step(s_x[0], a, s);
            stage_x_step(s_x[1], a, two ? s + 1 : s);
            load_tile_bf16(A, s, ra0);
            load_tile_bf16(A, two ? s + 1 : s, ra1);
            fence_schedule();
            wait_vm_all();  // this thread's copies and weights have landed
            staged_barrier();
#pragma unroll
            for (int c = 0; c < NCG; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[c] = mfma(as_bf16x8(ra0[j]), x_operand(s_x[0], c, j), acc[c]);
            if (two) {
#pragma unroll
                for (int c = 0; c < NCG; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[c] = mfma(as_bf16x8(ra1[j]), x_operand(s_x[1], c, j), acc[c]);
            }
        }
        // Partial sums of the slice, in MFMA layout: part[ks][t][c][lane];
        // router tiles token-major for the routing units: rpart[ks][b][e]
        // (lane (n, g) holds experts 16 tt + 4g .. + 3 of token 16c + n).
        if (active && kind == KIND_ROUTER) {
#pragma unroll
            for (int c = 0; c < NCG; ++c) {
                const int b = 16 * c + (lane & 15);
                if (b < a.B)
                    buf_st16<true>(rrpart, (uint32_t)((((size_t)ks * a.B + b) * kMaxExperts + 16 * tt + 4 * g) * 4),
                                   __builtin_bit_cast(u32x4, acc[c]));
            }
        } else if (active) {
#pragma unroll
            for (int c = 0; c < NCG; ++c)
                buf_st16<true>(rpart, (uint32_t)(((((size_t)ks * a.kx_tiles + t) * NCG + c) * kWave + lane) * 16),
                               __builtin_bit_cast(u32x4, acc[c]));
        }
        wait_vm_all();
        __syncthreads();
        uint32_t *rgc = a.rgc + (size_t)(a.dense_lo ? a.kx_groups : 0) * kCtrStride + (size_t)rg * kCtrStride;
        if (threadIdx.x == 0) {
            s_arrive = __hip_atomic_fetch_add(rgc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)nsl - 1u;
            // A router slice's partials are complete: the routing units add them.
            if (short_sl)
                __hip_atomic_fetch_add(&a.gctr[G_ROUTER_DONE], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_arrive) {  // the row group's last slice: sum the slices in order
            if (active && kind != KIND_ROUTER) {
                f32x4 sum[NCG];
                sum_slices<NCG>(rpart, nsl, a.kx_tiles, t, sum);
                dense_in_epilogue<false, NCG>(a, kind, tt, 0, sum, &s_last);
            }
            if (threadIdx.x == 0) store_agent(rgc, 0u);  // ready for the next step
        }
        __syncthreads();
    }
    if (a.kx_rg_r > 0)
        routing_units_tp(a, units, s_route, (float *)&s_x[0][0], &s_last);
    else
        routing_units(a, units, s_route, &s_last);
    prefetch_units(a, units + a.route_units);
}

// Kernel 2: gate/up units.  Late: the step's routing runs here first (at
// most kLatePairs pairs; the dense-in launch only stored scores and keys):
// every workgroup selects every token's experts and builds the unit records
// in LDS once, keeps the records of its own units (units blockIdx.x,
// blockIdx.x + gridDim.x, ..., at most kLateUnitsPerWG of them) in a small LDS
// array outside the staging buffer, and runs them.  The routing goes to global
// memory for the later launches: each column unit's record from the workgroup
// that runs its first tile group, everything else from workgroup 0.
constexpr int kLateUnitsPerWG = 16;
// Chunks of 8 steps (K split 1, not late) are compiled for three workgroups
// per compute unit (80 registers, 32 KB of LDS): with units of one workgroup
// each, more units in flight beat the longer weight burst of 16-step chunks
// that leave room for two (K3 batch 2 / 8 / 64 step: -3 / -3.4 / -3.2 %).
template <int S, bool Late, int KS = 1>
__global__ void __launch_bounds__(kWGThreads)
__attribute__((amdgpu_waves_per_eu(S == 8 && !Late && KS == 1 ? 6 : 4)))
k_w13(const StepArgs a) {
    constexpr int kStage = 8 * Stage<S>::kChunks * 2;
    constexpr int kBytes = Late && (int)sizeof(LateRouteLds) > kStage ? (int)sizeof(LateRouteLds)
                                                                       : kStage;
    __shared__ __attribute__((aligned(16))) char s_mem[kBytes];
    __shared__ int s_rec[Late ? kLateUnitsPerWG : 1][kRecWords];
    uint16_t *s_b = (uint16_t *)s_mem;
    constexpr int TW = kWG / KS;  // tiles per unit
    const int TG = ((a.I >> 3) + TW - 1) / TW;
    bool reuse = false;
    if constexpr (Late) {
        LateRouteLds &lds = *(LateRouteLds *)s_mem;
        const RouteArgs ra = route_args(a);
        route_late(ra, lds, blockIdx.x == 0);
        const int units = lds.ncols * TG;
        const int mine = units > (int)blockIdx.x
                             ? min(kLateUnitsPerWG, (units - (int)blockIdx.x + (int)gridDim.x - 1) /
                                                        (int)gridDim.x)
                             : 0;
        // Wave r copies (and, for a column unit's first tile group, publishes)
        // the record of the workgroup's unit r.
        const int lane = lane_id();
        for (int r = wave_index(); r < mine; r += kWG) {
            const int u = (int)blockIdx.x + r * (int)gridDim.x;
            const int c = u / TG;
            if (lane < kRecWords) {
                const int v = lds.rec[c][lane];
                s_rec[r][lane] = v;
                if (u % TG == 0) a.cu_rec[(size_t)c * kRecWords + lane] = v;
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.meta[M_N_COLS] = lds.ncols;
            a.meta[M_N_ACTIVE] = lds.n_active;
        }
        __syncthreads();  // the records are copied before the staging overwrites the image
        for (int r = 0; r < mine; ++r) {
            const int u = (int)blockIdx.x + r * (int)gridDim.x;
            const int recw = s_rec[r][lane & 31];
            w13_unit_rec<S, false, false, KS>(a, recw, u % TG, s_b, reuse);
        }
    } else {
        const int NC = min(load_agent(a.meta + M_N_COLS), a.ncols_cap);  // never beyond the records
        for (int u = blockIdx.x; u < NC * TG; u += gridDim.x) {
            int e, nt, p0;
            const int recw = read_record<false>(a, u / TG, e, nt, p0);
            w13_unit_rec<S, false, false, KS>(a, recw, u % TG, s_b, reuse);
        }
    }
}

// Kernel 3: down units (KS waves per tile; Ord: the ordered latent combine).
// Units of at most two steps (short experts) are latency-bound chains of a
// record read, the operand staging and the combine: four workgroups per
// compute unit keep more of them in flight (64 registers, no spills; TP8
// share batch 64: 140.7 -> 137.3 us per layer; the ordered form, whose
// pair stores need more registers, three).  Chunks of 8 steps (K split 1)
// take three workgroups, as in k_w13 (80 registers; the ordered form would
// spill).
template <int S, int KS, bool Ord = false>
__global__ void __launch_bounds__(kWGThreads)
__attribute__((amdgpu_waves_per_eu(S <= 2 && !Ord   ? 8
                                   : S <= 2 && KS == 1 ? 6
                                   : S == 8 && KS == 1 && !Ord ? 6
                                                              : 4)))
k_w2(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_b[8 * Stage<S>::kChunks];
    const int NC = min(load_agent(a.meta + M_N_COLS), a.ncols_cap);
    const int TG = ((a.L >> 4) + kWG / KS - 1) / (kWG / KS);
    bool reuse = false;
    for (int u = blockIdx.x; u < NC * TG; u += gridDim.x)
        w2_unit<S, false, KS, Ord>(a, u / TG, u % TG, s_b, reuse);
}

// Kernel 4 up to 8 tokens with column operands staged in LDS once per
// workgroup, instead of loaded (and, for ylat, split into hi/lo) by every wave
// at every step.  Full (up to kOutStTokens tokens): the whole reduction's
// operand, ylat split into hi/lo bf16 and then the shared activation's hi/lo
// rows (row 2b + part, L + Is elements).  Otherwise (up to 8 tokens): the
// ylat part only (L elements a row); the shared-down steps load their bf16
// operand from global memory with the weights, as k_out does.  The staging
// loads are issued before the wave's first two weight steps and waited for
// alone (vector loads complete in issue order), so their round trip overlaps
// the weight stream's.  A workgroup runs one output unit (the grid has one per
// unit); lanes without a token read the last staged row and their columns are
// dropped.
constexpr int kOutStTokens = 2;
constexpr int kOutStBytes = 2 * kOutStTokens * 6144 * 2;  // LDS limit of the full operand
constexpr int kOutStLatTokens = 8;
constexpr int kOutStLatBytes = 65536;                     // LDS limit of the ylat operand

// Weights of output step s: latent-up rows below Ls, shared-down rows above.
__device__ __forceinline__ void load_out_w(const TwoSource &t, int s, u32x4 (&ra)[4]) {
    if (s < t.Ls)
        load_tile_bf16(t.Aa, s, ra);
    else
        load_tile_bf16(t.Ab, s - t.Ls, ra);
}

__device__ __forceinline__ void mfma_tile_lds(const u32x4 (&ra)[4], const uint16_t *op, int s,
                                              f32x4 &acc) {
    const uint16_t *p = op + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma(as_bf16x8(ra[j]), as_bf16x8(*(const u32x4 *)(p + 32 * j)), acc);
}

template <bool Full>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_out_st(const StepArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t s_op[];  // [2B][KS]
    __shared__ float s_red[kWG * kWave * 4];
    if (blockIdx.x == 0 && threadIdx.x == 0) a.gctr[G_ROUTER_DONE] = 0u;
    const Role ro = role_of(a.kw_out);
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int KS = Full ? a.L + a.Is : a.L;  // staged elements per row
    const int RT = a.out_rows;
    const int n_t = (a.H + RT - 1) / RT;
    const int units = dense_units(n_t, ro.RW, 1);
    const int u = blockIdx.x;
    if (u >= units) return;
    int cb, tg;
    dense_unit(u, 1, cb, tg);
    const int t = tg * ro.RW + ro.rg;
    const bool active = t < n_t;
    // Staging loads: chunk q = 8 elements e .. e + 7 of token b (q < B KS / 8),
    // two 16-byte loads each (f32 ylat values, or the hi and the lo row of
    // the shared activation).
    const int nq = a.B * KS / 8;
    constexpr int kQ = ((Full ? kOutStBytes : kOutStLatBytes) / 32 + kWGThreads - 1) / kWGThreads;
    u32x4 st0[kQ], st1[kQ];
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int q = min((int)threadIdx.x + kWGThreads * i, nq - 1);
        const int b = q / (KS / 8), e = 8 * (q % (KS / 8));
        const bool lat = !Full || e < a.L;
        const uint8_t *p0 = lat ? (const uint8_t *)(a.ylat + (size_t)b * a.L + e)
                                : (const uint8_t *)(a.ashhl + (size_t)b * 2 * a.Is + (e - a.L));
        const uint8_t *p1 = lat ? p0 + 16 : p0 + (size_t)a.Is * 2;
        st0[i] = ld16(p0);
        st1[i] = ld16(p1);
    }
    fence_schedule();
    // The wave's first two weight steps, issued behind the staging loads.
    const int h0 = RT * (active ? t : 0);
    const size_t h = min(h0 + min(n, RT - 1), a.H - 1);
    TwoSource ts;
    ts.Aa = a.lat_up + h * a.L + 8 * g;
    ts.Ab = a.sh_w2 + h * a.Is + 8 * g;
    ts.Ls = a.L / kKStep;
    const int s0 = ro.kw * a.spc_out, s1 = s0 + a.spc_out;
    // Full: a ring of kXlRing weight steps in flight (every operand comes
    // from LDS, so the registers hold weights only); otherwise two steps.
    constexpr int kNw = Full ? kXlRing : 2;
    u32x4 rw[kNw][4];
#pragma unroll
    for (int i = 0; i < kNw; ++i) load_out_w(ts, min(s0 + i, s1 - 1), rw[i]);
    fence_schedule();
    // vmcnt(4 kNw): the staging loads have landed (vmcnt in bits [3:0] and [15:14]).
    __builtin_amdgcn_s_waitcnt(((4 * kNw) & 15) | (((4 * kNw) >> 4) << 14) | 0x0F70);
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int q = (int)threadIdx.x + kWGThreads * i;
        if (q < nq) {
            const int b = q / (KS / 8), e = 8 * (q % (KS / 8));
            u32x4 hi = st0[i], lo = st1[i];
            if (!Full || e < a.L) {  // f32 values: split into hi and lo bf16
                const f32x4 v0 = __builtin_bit_cast(f32x4, st0[i]), v1 = __builtin_bit_cast(f32x4, st1[i]);
                uint32_t hh[4], ll[4];
                split_hl2(v0[0], v0[1], hh[0], ll[0]);
                split_hl2(v0[2], v0[3], hh[1], ll[1]);
                split_hl2(v1[0], v1[1], hh[2], ll[2]);
                split_hl2(v1[2], v1[3], hh[3], ll[3]);
                hi = (u32x4){hh[0], hh[1], hh[2], hh[3]};
                lo = (u32x4){ll[0], ll[1], ll[2], ll[3]};
            }
            *(u32x4 *)(s_op + (size_t)(2 * b) * KS + e) = hi;
            *(u32x4 *)(s_op + (size_t)(2 * b + 1) * KS + e) = lo;
        }
    }
    lds_reuse_barrier();  // the staged operand is complete (weight loads still in flight)
    const uint16_t *op = s_op + (size_t)min(n, 2 * a.B - 1) * KS + 8 * g;
    // Shared-down operand from global memory (the ylat-only form).
    const bool valid = col < a.B;
    const rsrc_t rb_ash = buf_rsrc(a.ashhl);
    const uint32_t ob = (uint32_t)((((size_t)(valid ? col : 0) * 2 + part) * a.Is + 8 * g) * 2);
    f32x4 acc = zero4();
    if constexpr (Full) {
        if (active) {
#pragma unroll
            for (int i = 0; i < kMaxStepsPerChunk; ++i) {
                if (i < a.spc_out) {
                    mfma_tile_lds(rw[i % kNw], op, s0 + i, acc);
                    if (i + kNw < a.spc_out) load_out_w(ts, s0 + i + kNw, rw[i % kNw]);
                }
            }
        }
    } else if (active) {
        u32x4(&ra0)[4] = rw[0];
        u32x4(&ra1)[4] = rw[1 % kNw];
#pragma unroll 1
        for (int s = s0; s < s1; s += 2) {
            const bool two = s + 1 < s1;
            const int s2 = two ? s + 1 : s;
            if (s > s0) {
                load_out_w(ts, s, ra0);
                load_out_w(ts, s2, ra1);
            }
            u32x4 rb0[4], rb1[4];
            if (s >= ts.Ls) buf_cols_bf16<false>(rb_ash, ob, valid, s - ts.Ls, rb0);
            if (s2 >= ts.Ls) buf_cols_bf16<false>(rb_ash, ob, valid, s2 - ts.Ls, rb1);
            fence_schedule();
            if (s < ts.Ls)
                mfma_tile_lds(ra0, op, s, acc);
            else
                mfma_tile(ra0, rb0, acc);
            if (two) {
                if (s2 < ts.Ls)
                    mfma_tile_lds(ra1, op, s2, acc);
                else
                    mfma_tile(ra1, rb1, acc);
            }
        }
    }
    const bool leader = reduce_k1(s_red, ro.wave, ro.kw, ro.KW, acc);
    if (leader && active) {
        const f32x4 v = add_pair_column(acc);
        if (col < a.B && part == 0) {
            const size_t o = (size_t)col * a.H + h0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i;
                if (r < RT && h0 + r < a.H) a.out[o + r] = (uint16_t)bf16_rne(v[i]);
            }
        }
    }
}

// Kernel 4: output units (latent-up and shared-down in one pass), each over
// NCG column groups of 8 tokens: ceil(ceil(B / 8) / NCG) units per tile.
template <int NCG>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_out(const StepArgs a) {
    __shared__ float s_red[NCG * kWG * kWave * 4];
    // The router counter of the dense input kernel is cleared here, where no
    // wave of the step can touch it any more.
    if (blockIdx.x == 0 && threadIdx.x == 0) a.gctr[G_ROUTER_DONE] = 0u;
    const Role ro = role_of(a.kw_out);
    const int nblk = (((a.B + 7) >> 3) + NCG - 1) / NCG;
    const int n_t = (a.H + a.out_rows - 1) / a.out_rows;
    const int units = dense_units(n_t, ro.RW, nblk);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int cb, tg;
        dense_unit(u, nblk, cb, tg);
        const int t = tg * ro.RW + ro.rg;
        out_tile_n<NCG>(a, ro, t, t < n_t, cb * NCG, s_red);
    }
}

// Kernel 4 for more than 8 tokens (NCG in {2, 4, 8} column groups of 8
// tokens), built like k_dense_in_kx: a unit is 8 output tiles (one per wave)
// times a K slice of a.kx_sps_out steps.  Per pair of steps the workgroup
// copies every token's column operand into LDS once: ylat as f32 at
// latent-up steps (64 rows of 128 values; each lane splits its values into
// the hi or lo half when it reads them) and the hi/lo rows of the shared
// activation at shared-down steps (128 rows of 128 bf16).  Each slice adds
// every token's hi and lo columns before it stores its partial sums (half the
// partial bytes) and arrives on its row group's counter; sum units after the
// slices in the grid add the partials in slice order and round to bf16 once.
constexpr int kOutStage = 32768;  // bytes of one staged step (both kinds)

__device__ __forceinline__ void stage_out_step(char *buf, const StepArgs &a, int s, int Ls) {
    const int lane = lane_id(), wave = wave_index();
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int c0 = 64 * (wave + kWG * h), c = c0 + lane;  // 16-byte chunk 0 .. 2047
        const void *gp;
        if (s < Ls) {
            // ylat row b (32 chunks of 4 f32), chunk q at position q ^ 2(b & 7)
            const int b = c >> 5, q = (c & 31) ^ (2 * (b & 7));
            gp = a.ylat + (size_t)(b < a.B ? b : 0) * a.L + (size_t)s * kKStep + 4 * q;
        } else {
            // ash row r = 2b + part (16 chunks of 8 bf16), chunk q at q ^ (r & 15)
            const int r = c >> 4, b = r >> 1, q = (c & 15) ^ (r & 15);
            gp = a.ashhl + ((size_t)(b < a.B ? b : 0) * 2 + (r & 1)) * a.Is +
                 (size_t)(s - Ls) * kKStep + 8 * q;
        }
        __builtin_amdgcn_global_load_lds(gp, buf + 16 * c0, 16, 0, 0);
    }
}

// Turns a staged ylat step (f32 rows) in place into the layout of a staged
// shared-activation step: row 2b + part holds token b's hi (part 0) or lo
// (part 1) bf16 halves, chunk q at position q ^ (row & 15).  Thread i takes
// token i / 8 and its 16 values [16 (i % 8), + 16): all read, then all
// write.  Starts and ends with a workgroup barrier.
__device__ __forceinline__ void ylat_to_hl(char *buf) {
    const int i = threadIdx.x, b = i >> 3, e0 = 16 * (i & 7), sw = 2 * (b & 7);
    const float *row = (const float *)(buf + b * (kKStep * 4));
    f32x4 v[4];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) v[m] = *(const f32x4 *)(row + 4 * (((e0 >> 2) + m) ^ sw));
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        split_hl2(v[m][0], v[m][1], hi[2 * m], lo[2 * m]);
        split_hl2(v[m][2], v[m][3], hi[2 * m + 1], lo[2 * m + 1]);
    }
    __syncthreads();
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        const int r = 2 * b + part;
        const uint32_t *w = part ? lo : hi;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = (e0 >> 3) + h;  // 8 bf16 per chunk
            *(u32x4 *)(buf + r * (kKStep * 2) + 16 * (q ^ (r & 15))) =
                (u32x4){w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
        }
    }
    __syncthreads();
}

// MFMA j's column operand of group c from a staged step in the hi/lo row
// layout: lane (n, g) takes row 16c + n (token 8c + n/2, hi for n even, lo
// for n odd), elements [32j + 8g, 32j + 8g + 8).
__device__ __forceinline__ bf16x8 out_operand(const char *buf, int c, int j) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int r = 16 * c + n;
    return as_bf16x8(*(const u32x4 *)(buf + r * (kKStep * 2) + 16 * ((4 * j + g) ^ n)));
}

template <int NCG>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_out_kx(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) char s_o[2][kOutStage];
    // The router counter of the dense input kernel is cleared here, as in k_out.
    if (blockIdx.x == 0 && threadIdx.x == 0) a.gctr[G_ROUTER_DONE] = 0u;
    const int lane = lane_id(), wave = wave_index(), n = lane & 15, g = lane >> 4;
    const int RT = a.out_rows, n_ot = (a.H + RT - 1) / RT;
    const int Ls = a.L / kKStep, nsteps = Ls + a.Is / kKStep;
    const int sps = a.kx_sps_out, nsl = (nsteps + sps - 1) / sps;
    const int units = ((n_ot + kWG - 1) / kWG) * nsl;
    const rsrc_t rpart = buf_rsrc(a.part);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int rg = u / nsl, ks = u % nsl;
        const int t = rg * kWG + wave;
        const bool active = t < n_ot;
        const int h0 = RT * (active ? t : 0);
        const size_t h = min(h0 + min(n, RT - 1), a.H - 1);
        const uint16_t *Aa = a.lat_up + h * a.L + 8 * g, *Ab = a.sh_w2 + h * a.Is + 8 * g;
        const int s0 = ks * sps, s1 = min(nsteps, s0 + sps);
        f32x4 acc[NCG];
#pragma unroll
        for (int c = 0; c < NCG; ++c) acc[c] = zero4();
        for (int s = s0; s < s1; s += 2) {
            const int s2 = s + 1 < s1 ? s + 1 : s;
            __syncthreads();  // every wave is done with the staged copies
            u32x4 ra0[4], ra1[4];
            stage_out_step(s_o[0], a, s, Ls);
            stage_out_step(s_o[1], a, s2, Ls);
            if (s < Ls) load_tile_bf16(Aa, s, ra0); else load_tile_bf16(Ab, s - Ls, ra0);
            if (s2 < Ls) load_tile_bf16(Aa, s2, ra1); else load_tile_bf16(Ab, s2 - Ls, ra1);
            fence_schedule();
            wait_vm_all();  // this thread's copies and weights have landed
            staged_barrier();
            if (s < Ls) ylat_to_hl(s_o[0]);
            if (s2 != s && s2 < Ls) ylat_to_hl(s_o[1]);
#pragma unroll
            for (int c = 0; c < NCG; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[c] = mfma(as_bf16x8(ra0[j]), out_operand(s_o[0], c, j), acc[c]);
            if (s2 != s) {
#pragma unroll
                for (int c = 0; c < NCG; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[c] = mfma(as_bf16x8(ra1[j]), out_operand(s_o[1], c, j), acc[c]);
            }
        }
        // Partial sums of the slice with each token's hi and lo columns
        // added, two column groups per store: lane (n, g) holds group 2c + (n
        // & 1), token column n / 2: part[ks][t][c][lane], c < NCG / 2.
        if (active) {
#pragma unroll
            for (int c = 0; c < NCG / 2; ++c) {
                const f32x4 v0 = add_pair_column(acc[2 * c]), v1 = add_pair_column(acc[2 * c + 1]);
                buf_st16<true>(rpart, (uint32_t)(((((size_t)ks * n_ot + t) * (NCG / 2) + c) * kWave + lane) * 16),
                               __builtin_bit_cast(u32x4, (n & 1) ? v1 : v0));
            }
        }
        wait_vm_all();
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(a.rgc + (size_t)rg * kCtrStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    // Sum units, after the slice units in the grid (so dispatched only once
    // every slice unit has been): unit s adds, in slice order, the partial
    // sums of tiles 8 rg + 4 h .. + 3 (rg = s / 2, h = s % 2) once all nsl
    // slices of row group rg have arrived, and rounds to bf16 once.  Thread
    // i takes chunks i and i + 512 of the half's 4 tiles x NCG / 2 groups x
    // 64 lanes: every slice's load in one round trip (the slices' last
    // arrival summing all 8 tiles took two).
    constexpr int kSumChunks = 4 * (NCG / 2) * kWave;
    constexpr int kSumPer = (kSumChunks + kWGThreads - 1) / kWGThreads;
    const int nrg = (n_ot + kWG - 1) / kWG;
    for (int su = (int)blockIdx.x - units; su >= 0 && su < 2 * nrg; su += gridDim.x) {
        const int rg = su >> 1, hf = su & 1;
        uint32_t *rgc = a.rgc + (size_t)rg * kCtrStride;
        wg_wait(a, rgc, (uint32_t)nsl);
        u32x4 v[kSumPer][kMaxSlicesOut];
#pragma unroll
        for (int q = 0; q < kSumPer; ++q) {
            const int x = min((int)threadIdx.x + kWGThreads * q, kSumChunks - 1);
            const int t = min(kWG * rg + 4 * hf + x / ((NCG / 2) * kWave), n_ot - 1);
            const int c = (x / kWave) % (NCG / 2), l = x % kWave;
#pragma unroll
            for (int k = 0; k < kMaxSlicesOut; ++k) {
                const int kk = min(k, nsl - 1);
                v[q][k] = buf_ld16<true>(rpart, (uint32_t)(((((size_t)kk * n_ot + t) * (NCG / 2) + c) * kWave + l) * 16));
            }
        }
#pragma unroll
        for (int q = 0; q < kSumPer; ++q) {
            const int x = (int)threadIdx.x + kWGThreads * q;
            const int t = kWG * rg + 4 * hf + x / ((NCG / 2) * kWave);
            const int c = (x / kWave) % (NCG / 2), l = x % kWave, ln = l & 15, lg = l >> 4;
            f32x4 sum = zero4();
#pragma unroll
            for (int k = 0; k < kMaxSlicesOut; ++k)
                if (k < nsl) sum += __builtin_bit_cast(f32x4, v[q][k]);
            const int b = 8 * (2 * c + (ln & 1)) + (ln >> 1), h0 = RT * t;
            if (x < kSumChunks && t < n_ot && b < a.B) {
                const size_t o = (size_t)b * a.H + h0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lg + i;
                    if (r < RT && h0 + r < a.H) a.out[o + r] = (uint16_t)bf16_rne(sum[i]);
                }
            }
        }
        // Each half arrives once more after its wait; the second resets the
        // counter for the next step.
        if (threadIdx.x == 0 &&
            __hip_atomic_fetch_add(rgc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)nsl + 1u)
            store_agent(rgc, 0u);
    }
}

// Output kernels of the side-stream step: shared-down (MODE = OUT_SHARED,
// f32 sums to ysh, on the side stream) and latent-up (MODE = OUT_LATENT,
// adds ysh, one bf16 rounding, on the caller's stream after the join); one
// column group of 8 tokens per unit.
template <int MODE>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_out_part(const StepArgs a) {
    __shared__ float s_red[kWG * kWave * 4];
    // The latent-up launch ends the step: it clears the router counter of the
    // dense input kernel, as k_out does.
    if (MODE == OUT_LATENT && blockIdx.x == 0 && threadIdx.x == 0) a.gctr[G_ROUTER_DONE] = 0u;
    const Role ro = role_of(MODE == OUT_SHARED ? a.kw_sd : a.kw_lu);
    const int spc = MODE == OUT_SHARED ? a.spc_sd : a.spc_lu;
    const int ncg = (a.B + 7) >> 3;
    const int n_t = (a.H + a.out_rows - 1) / a.out_rows;
    const int units = dense_units(n_t, ro.RW, ncg);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int cg, tg;
        dense_unit(u, ncg, cg, tg);
        const int t = tg * ro.RW + ro.rg;
        out_tile<false>(a, ro, MODE, t, t < n_t, cg, spc, s_red);
    }
}

// ---------------------------------------------------------------------------
// Fused step: one persistent launch
// ---------------------------------------------------------------------------
//
// The units of the step form one list in dependency order:
//   [router | latent-down | shared gate/up | gate/up | down | shared-down |
//    latent-up]
// (ranges a.u_*).  Workgroups take units from an agent-scope counter, so a
// taken unit always belongs to a running workgroup; a unit waits only for
// units earlier in the list, hence the step always progresses, whether or not
// the whole grid is resident.  A
// unit's outputs are published with agent-scope stores, then one counter
// increment; a waiting unit polls the counter from one lane (bounded: after
// kSpinLimit polls it records G_ERROR and goes on instead of hanging).  The
// last workgroup to leave the queue resets every counter for the next step.

// Active column units of the step (known once the routing has published).
__device__ __forceinline__ int routed_units(const StepArgs &a) {
    wg_wait(a, &a.gctr[G_ROUTED], 1u);
    return min(load_agent(a.meta + M_N_COLS), a.ncols_cap);
}

template <int S13, int S2>
struct StepLds {
    static constexpr int kExpert = 8 * Stage<(S13 > S2 ? S13 : S2)>::kChunks * 2;
    static constexpr int kDense = (int)sizeof(RouteLds) + kWG * kWave * 4 * 4;
    static constexpr int kBytes = kExpert > kDense ? kExpert : kDense;
};

template <int S13, int S2>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_step(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) char s_mem[StepLds<S13, S2>::kBytes];
    __shared__ int s_last, s_next, s_exit;
    RouteLds *s_route = (RouteLds *)s_mem;
    float *s_red = (float *)(s_mem + sizeof(RouteLds));
    float *s_red_out = (float *)s_mem;
    uint16_t *s_b = (uint16_t *)s_mem;
    const Role ro_in = role_of(a.kw_in), ro_sd = role_of(a.kw_sd), ro_lu = role_of(a.kw_lu);
    const int ncg_in = (a.B + 15) >> 4, ncg_out = (a.B + 7) >> 3;
    const int n_lt = a.L / a.latent_rows, n_st = a.Is >> 3;
    const int n_ot = (a.H + a.out_rows - 1) / a.out_rows;
    if (threadIdx.x == 0) {
        s_last = 0;
        s_next = (int)__hip_atomic_fetch_add(&a.gctr[G_WORK], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    int u = s_next;
    while (u < a.u_end) {
        if (u < a.u_sh) {
            // router or latent-down unit
            const bool router = u < a.u_lat;
            const int ui = router ? u : u - a.u_lat;
            const int cg = ui % ncg_in, t = (ui / ncg_in) * ro_in.RW + ro_in.rg;
            const int n_kind = router ? a.n_rtiles : n_lt;
            if (!router) {
                // This unit's slice of ylat goes to zero before any down unit
                // can add to it (they wait for every latent unit).
                const int n4 = a.B * a.L / 4, per = (n4 + a.n_lat_units - 1) / a.n_lat_units;
                for (int i = ui * per + (int)threadIdx.x; i < min(n4, (ui + 1) * per); i += kWGThreads) {
                    uint64_t *q = (uint64_t *)(a.ylat + 4 * i);
                    __hip_atomic_store(q, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(q + 1, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            dense_in_tile<true>(a, ro_in, router ? KIND_ROUTER : KIND_LATENT, t, t < n_kind, cg, s_red,
                          &s_last);
            if (router) {
                if (s_last) {  // this workgroup completed the router: route the step
                    route_step<true>(route_args(a), s_route, kWG);
                    if (threadIdx.x == 0) s_last = 0;
                    wg_publish(&a.gctr[G_ROUTED]);
                }
            } else {
                wg_publish(&a.gctr[G_LATENT]);
            }
        } else if (u < a.u_13) {
            // shared gate/up unit
            const int ui = u - a.u_sh;
            const int cg = ui % ncg_in, t = (ui / ncg_in) * ro_in.RW + ro_in.rg;
            dense_in_tile<true>(a, ro_in, KIND_SHARED, t, t < n_st, cg, s_red, &s_last);
            wg_publish(&a.gctr[G_SHARED]);
        } else if (u < a.u_2) {
            // gate/up unit: needs the routing and every z row
            const int ui = u - a.u_13, c = ui / a.tg13;
            if (c < routed_units(a)) {
                wg_wait(a, &a.gctr[G_LATENT], (uint32_t)a.n_lat_units);
                bool reuse = true;
                w13_unit<S13, true, true>(a, c, ui % a.tg13, s_b, reuse);
                wg_publish(&a.c13[c * kCtrStride]);
            }
        } else if (u < a.u_sd) {
            // down unit: needs its column unit's activations
            const int ui = u - a.u_2, c = ui / a.tg2;
            if (c < routed_units(a)) {
                wg_wait(a, &a.c13[c * kCtrStride], (uint32_t)a.tg13);
                bool reuse = true;
                w2_unit<S2, true>(a, c, ui % a.tg2, s_b, reuse);
                wg_publish(&a.gctr[G_W2]);
            }
        } else if (u < a.u_lu) {
            // shared-down unit: needs every shared activation
            const int ui = u - a.u_sd;
            const int cg = ui % ncg_out, t = (ui / ncg_out) * ro_sd.RW + ro_sd.rg;
            wg_wait(a, &a.gctr[G_SHARED], (uint32_t)a.n_sh_units);
            out_tile<true>(a, ro_sd, OUT_SHARED, t, t < n_ot, cg, a.spc_sd, s_red_out);
            wg_publish(&a.gctr[G_SHDOWN]);
        } else {
            // latent-up unit: needs the whole latent combine and the
            // shared-down sums
            const int ui = u - a.u_lu;
            const int cg = ui % ncg_out, t = (ui / ncg_out) * ro_lu.RW + ro_lu.rg;
            const int NC = routed_units(a);
            wg_wait(a, &a.gctr[G_W2], (uint32_t)(NC * a.tg2));
            wg_wait(a, &a.gctr[G_SHDOWN], (uint32_t)a.n_sd_units);
            out_tile<true>(a, ro_lu, OUT_LATENT, t, t < n_ot, cg, a.spc_lu, s_red_out);
        }
        // The next unit is taken only now: a unit taken while another one
        // still waits would hold up the units that depend on it.
        __syncthreads();
        if (threadIdx.x == 0)
            s_next = (int)__hip_atomic_fetch_add(&a.gctr[G_WORK], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        u = s_next;
    }
    // The last workgroup out of the queue resets the counters: no other
    // workgroup of this launch touches them any more.
    if (threadIdx.x == 0)
        s_exit = __hip_atomic_fetch_add(&a.gctr[G_EXIT], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u;
    __syncthreads();
    if (s_exit) {
        for (int i = threadIdx.x; i < G_ERROR; i += kWGThreads)
            __hip_atomic_store(&a.gctr[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = threadIdx.x; i < a.ncols_cap; i += kWGThreads)
            __hip_atomic_store(&a.c13[i * kCtrStride], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Two-launch step: the dense-in kernel (router, routing, latent-down, shared
// gate/up), then one persistent launch for the rest
// ---------------------------------------------------------------------------
//
// The second launch runs the units
//   [gate/up (NC x tg13) | shared-down, first part | down (NC x tg2) |
//    shared-down, rest | latent-up]
// from one queue in this order, NC being the routing's active column units.
// The shared-down units depend on nothing in this launch: placed between the
// dependent phases, they keep the compute units streaming weights while the
// down units wait for their column's gate/up units and the latent-up units
// for the whole latent combine.  The same progress argument as the fused
// step holds (a unit waits only for units earlier in the queue).

template <int S13, int S2>
struct TailLds {
    static constexpr int kExpert = 8 * Stage<(S13 > S2 ? S13 : S2)>::kChunks * 2;
    static constexpr int kOut = kWG * kWave * 4 * 4;
    static constexpr int kBytes = kExpert > kOut ? kExpert : kOut;
};

template <int S13, int S2>
__global__ void __launch_bounds__(kWGThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_tail(const StepArgs a) {
    __shared__ __attribute__((aligned(16))) char s_mem[TailLds<S13, S2>::kBytes];
    __shared__ int s_next, s_exit;
    uint16_t *s_b = (uint16_t *)s_mem;
    float *s_red = (float *)s_mem;
    const Role ro_sd = role_of(a.kw_sd), ro_lu = role_of(a.kw_lu);
    const int ncg_out = (a.B + 7) >> 3;
    const int n_ot = (a.H + a.out_rows - 1) / a.out_rows;
    // Written by the dense-in launch; never beyond the records.
    const int NC = min(a.meta[M_N_COLS], a.ncols_cap);
    const int r13 = NC * a.tg13, rsa = r13 + a.n_sd_first, r2 = rsa + NC * a.tg2;
    const int rsb = r2 + (a.n_sd_units - a.n_sd_first), rend = rsb + a.n_lu_units;
    if (threadIdx.x == 0)
        s_next = (int)__hip_atomic_fetch_add(&a.gctr[G_WORK], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int u = s_next;
    while (u < rend) {
        if (u < r13) {
            // gate/up unit: z and the records come from the dense-in launch
            const int c = u / a.tg13;
            bool reuse = true;
            w13_unit<S13, false, true>(a, c, u % a.tg13, s_b, reuse);
            wg_publish(&a.c13[c * kCtrStride]);
        } else if (u < rsa || (u >= r2 && u < rsb)) {
            // shared-down unit: the shared activation comes from the dense-in
            // launch
            const int ui = u < rsa ? u - r13 : a.n_sd_first + (u - r2);
            const int cg = ui % ncg_out, t = (ui / ncg_out) * ro_sd.RW + ro_sd.rg;
            out_tile<false>(a, ro_sd, OUT_SHARED, t, t < n_ot, cg, a.spc_sd, s_red);
            wg_publish(&a.gctr[G_SHDOWN]);
        } else if (u < r2) {
            // down unit: needs its column unit's activations
            const int ui = u - rsa, c = ui / a.tg2;
            wg_wait(a, &a.c13[c * kCtrStride], (uint32_t)a.tg13);
            bool reuse = true;
            w2_unit<S2, true>(a, c, ui % a.tg2, s_b, reuse);
            wg_publish(&a.gctr[G_W2]);
        } else {
            // latent-up unit: needs the whole latent combine and the
            // shared-down sums
            const int ui = u - rsb;
            const int cg = ui % ncg_out, t = (ui / ncg_out) * ro_lu.RW + ro_lu.rg;
            wg_wait(a, &a.gctr[G_W2], (uint32_t)(NC * a.tg2));
            wg_wait(a, &a.gctr[G_SHDOWN], (uint32_t)a.n_sd_units);
            out_tile<true>(a, ro_lu, OUT_LATENT, t, t < n_ot, cg, a.spc_lu, s_red);
        }
        __syncthreads();
        if (threadIdx.x == 0)
            s_next = (int)__hip_atomic_fetch_add(&a.gctr[G_WORK], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        u = s_next;
    }
    // The last workgroup out resets the counters of both launches.
    if (threadIdx.x == 0)
        s_exit = __hip_atomic_fetch_add(&a.gctr[G_EXIT], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u;
    __syncthreads();
    if (s_exit) {
        for (int i = threadIdx.x; i < G_ERROR; i += kWGThreads)
            __hip_atomic_store(&a.gctr[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = threadIdx.x; i < NC; i += kWGThreads)
            __hip_atomic_store(&a.c13[i * kCtrStride], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
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
