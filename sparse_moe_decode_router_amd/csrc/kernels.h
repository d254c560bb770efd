// kernels.h - the decode-step kernels for gfx950 (MI355X).
//
// Every contraction of the step is an HBM-bound matrix-vector / small-matrix
// product: weight rows are the 16-row A operand of v_mfma_f32_16x16x32_bf16,
// tokens are its 16 B columns.  The step is four launches (five with an f32
// router):
//   k_dense_in : router logits, latent-down z = W_ld x and shared gate/up
//                (all contract over the hidden size H against x); epilogues:
//                sigmoid + bias keys, z as hi/lo bf16, shared SwiGLU.  The
//                router tiles come first and the top-k + routing metadata run
//                inside this kernel while the latent and shared rows stream.
//   k_w13      : active experts' MXFP4 gate/up rows, fused dequantisation,
//                SwiGLU epilogue -> expert activation a (hi/lo bf16).
//   k_w2       : active experts' MXFP4 down rows; the last arrival for a
//                32-row latent tile forms the weighted combine ylat.
//   k_out      : latent-up W_lu ylat plus shared-down S2 ash, one bf16 RNE.
//
// Work decomposition.  A unit is one wave: 32 weight rows (two 16-row MFMA
// tiles) x one K chunk x one column group of tokens.  Units are split along K
// so that there are several thousand of them (256 CUs, 8 XCDs); each unit
// writes an f32 partial and arrives on a per-tile counter, and the last
// arrival sums the partials in chunk order (deterministic) and runs the
// epilogue.  No wave waits for another.
//
// Operands.  x is bf16 and enters the MFMA as is (16 tokens per column group).
// f32 intermediates (z, a, ylat, ash) are stored as hi + lo bf16 and enter as
// two adjacent columns of the same MFMA (8 tokens per column group); the two
// column sums are added afterwards, which keeps f32-grade precision at the cost
// of one MFMA per K-slice.
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

// ---------------------------------------------------------------------------
// Dense bf16 rows x bf16 tokens (router, latent-down, shared gate/up)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load_rows_bf16(const uint16_t *A0, const uint16_t *A1, int s,
                                               u32x4 (&ra)[8]) {
    const uint16_t *p0 = A0 + (size_t)s * kKStep;
    const uint16_t *p1 = A1 + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ra[j] = ld_weight16(p0 + 8 * j);
        ra[4 + j] = ld_weight16(p1 + 8 * j);
    }
}

// Column operand of one step.  Lanes without a token read a valid row (the
// caller points them at one) and drop the value, so no load sits under a
// lane-dependent branch.
__device__ __forceinline__ void load_cols(const uint16_t *X, bool valid, int s, u32x4 (&rb)[4]) {
    const uint16_t *p = X + (size_t)s * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 v = ld16(p + 8 * j);
        rb[j] = valid ? v : (u32x4){0u, 0u, 0u, 0u};
    }
}

// acc0/acc1 += rows A0/A1 (16 each) . columns X over the SPC steps from s0,
// with the next step's loads in flight while the current step's MFMAs run.
template <int SPC>
__device__ __forceinline__ void dense_chunk(const uint16_t *A0, const uint16_t *A1,
                                            const uint16_t *X, bool valid, int s0, f32x4 &acc0,
                                            f32x4 &acc1) {
    u32x4 ra[2][8], rb[2][4];
    load_rows_bf16(A0, A1, s0, ra[0]);
    load_cols(X, valid, s0, rb[0]);
#pragma unroll
    for (int q = 0; q < SPC; ++q) {
        if (q + 1 < SPC) {
            load_rows_bf16(A0, A1, s0 + q + 1, ra[(q + 1) & 1]);
            load_cols(X, valid, s0 + q + 1, rb[(q + 1) & 1]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 b = as_bf16x8(rb[q & 1][j]);
            acc0 = mfma(as_bf16x8(ra[q & 1][j]), b, acc0);
            acc1 = mfma(as_bf16x8(ra[q & 1][4 + j]), b, acc1);
        }
    }
}

// Same for the output kernel: K runs over [0, L) against lat_up and ylat,
// then over [0, Is) against sh_w2 and ash.  Step s < Ls selects the first pair.
struct TwoSource {
    const uint16_t *A0a, *A1a, *Xa;  // K in [0, L)
    const uint16_t *A0b, *A1b, *Xb;  // K in [0, Is)
    int Ls;                          // L / 128
};

__device__ __forceinline__ void load_two(const TwoSource &t, bool valid, int s, u32x4 (&ra)[8],
                                         u32x4 (&rb)[4]) {
    const bool first = s < t.Ls;
    const int ss = first ? s : s - t.Ls;
    load_rows_bf16(first ? t.A0a : t.A0b, first ? t.A1a : t.A1b, ss, ra);
    load_cols(first ? t.Xa : t.Xb, valid, ss, rb);
}

template <int SPC>
__device__ __forceinline__ void out_chunk(const TwoSource &t, bool valid, int s0, f32x4 &acc0,
                                          f32x4 &acc1) {
    u32x4 ra[2][8], rb[2][4];
    load_two(t, valid, s0, ra[0], rb[0]);
#pragma unroll
    for (int q = 0; q < SPC; ++q) {
        if (q + 1 < SPC) load_two(t, valid, s0 + q + 1, ra[(q + 1) & 1], rb[(q + 1) & 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 b = as_bf16x8(rb[q & 1][j]);
            acc0 = mfma(as_bf16x8(ra[q & 1][j]), b, acc0);
            acc1 = mfma(as_bf16x8(ra[q & 1][4 + j]), b, acc1);
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 expert rows x hi/lo token columns
// ---------------------------------------------------------------------------

// acc0/acc1 += MXFP4 rows (q0,sc0)/(q1,sc1) . columns X over the SPC steps
// from s0.  All code and scale loads of the chunk (2 x SPC x 16 code bytes
// and 2 x SPC scale dwords per lane) are issued first; the column operand is
// fetched one step ahead.  q0/q1 point at the lane's 16-byte slice of step 0,
// sc0/sc1 at the row's scale bytes (byte 4s+g is lane group g's block).
template <int SPC>
__device__ __forceinline__ void fp4_chunk(const uint8_t *q0, const uint8_t *sc0,
                                          const uint8_t *q1, const uint8_t *sc1,
                                          const uint16_t *X, bool valid, int g, int s0,
                                          f32x4 &acc0, f32x4 &acc1) {
    u32x4 c0[SPC], c1[SPC];
    uint32_t e0[SPC], e1[SPC];
    u32x4 rb[2][4];
    load_cols(X, valid, s0, rb[0]);
#pragma unroll
    for (int q = 0; q < SPC; ++q) {
        c0[q] = ld_weight16(q0 + (size_t)(s0 + q) * 64);
        c1[q] = ld_weight16(q1 + (size_t)(s0 + q) * 64);
        e0[q] = ld_weight4(sc0 + (size_t)(s0 + q) * 4);
        e1[q] = ld_weight4(sc1 + (size_t)(s0 + q) * 4);
    }
    const int sh = 8 * g;
#pragma unroll
    for (int q = 0; q < SPC; ++q) {
        if (q + 1 < SPC) load_cols(X, valid, s0 + q + 1, rb[(q + 1) & 1]);
        const float f0 = e8m0_scale((e0[q] >> sh) & 0xFFu);
        const float f1 = e8m0_scale((e1[q] >> sh) & 0xFFu);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 b = as_bf16x8(rb[q & 1][j]);
            acc0 = mfma(fp4x8_to_bf16(c0[q][j], f0), b, acc0);
            acc1 = mfma(fp4x8_to_bf16(c1[q][j], f1), b, acc1);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 0 (f32 router only): logits, scores and keys with plain f32 FMAs.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kBlock) k_router_f32(const StepArgs a) {
    __shared__ unsigned long long s_mask[kMaxExperts];
    const int lane = lane_id();
    const int nwaves = gridDim.x * kWavesPerBlock;
    for (int e = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); e < a.E; e += nwaves) {
        const float *row = a.router_w32 + (size_t)e * a.H;
        for (int b = 0; b < a.B; ++b) {
            const uint16_t *xb = a.x + (size_t)b * a.H;
            float acc = 0.f;
            for (int h = lane; h < a.H; h += kWave) acc = fmaf(row[h], bf16_val(xb[h]), acc);
            acc = wave_sum(acc);
            if (lane == 0) {
                const float s = sigmoidf_(acc);
                a.score[(size_t)b * a.E + e] = s;
                a.key[(size_t)b * a.E + e] = s + (a.bias ? a.bias[e] : 0.f);
            }
        }
        if (wave_arrive(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u)
            topk_loop(a, s_mask);
        else
            maybe_join_topk(a, s_mask);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1: router + latent-down + shared gate/up over x.
// ---------------------------------------------------------------------------

template <int SPC>
__global__ void __launch_bounds__(kBlock) k_dense_in(const StepArgs a) {
    __shared__ unsigned long long s_mask[kMaxExperts];
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int n_l2 = a.L >> 5, n_s2 = a.Is >> 4;
    const int n_t2 = a.n_r2 + n_l2 + n_s2;
    const int ncg = (a.B + 15) >> 4;
    const int total = n_t2 * ncg * a.s_in;
    const int nwaves = gridDim.x * kWavesPerBlock;
    for (int u = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); u < total; u += nwaves) {
        const int c = u % a.s_in, r = u / a.s_in, cg = r % ncg, t2 = r / ncg;
        const int s0 = c * SPC;
        int kind;
        const uint16_t *A0, *A1;
        if (t2 < a.n_r2) {
            kind = 0;
            A0 = a.router_w + (size_t)(32 * t2 + n) * a.H;
            A1 = A0 + (size_t)16 * a.H;
        } else if (t2 < a.n_r2 + n_l2) {
            kind = 1;
            A0 = a.lat_down + (size_t)(32 * (t2 - a.n_r2) + n) * a.H;
            A1 = A0 + (size_t)16 * a.H;
        } else {
            kind = 2;
            const int pt = t2 - a.n_r2 - n_l2;
            A0 = a.sh_w13 + (size_t)(16 * pt + n) * a.H;
            A1 = a.sh_w13 + (size_t)(a.Is + 16 * pt + n) * a.H;
        }
        const int b = 16 * cg + n;
        const bool valid = b < a.B;
        const uint16_t *X = a.x + (size_t)(valid ? b : 0) * a.H + 32 * g;
        f32x4 acc0 = zero4(), acc1 = zero4();
        dense_chunk<SPC>(A0 + 32 * g, A1 + 32 * g, X, valid, s0, acc0, acc1);

        bool finish = true;
        if (a.s_in > 1) {
            float *mine = a.part_in + ((size_t)(t2 * a.s_in + c) * a.Bm + b) * 32 + 4 * g;
            if (valid) {
                stf4(mine, acc0);
                stf4(mine + 16, acc1);
            }
            uint32_t *ctr = a.ctr_in + t2 * a.ncg_in_cap + cg;
            finish = wave_arrive(ctr) == (uint32_t)(a.s_in - 1);
            if (finish) {
                acquire_agent();
                wave_store_counter(ctr, 0u);
                acc0 = zero4();
                acc1 = zero4();
                if (valid) {
                    const float *p = a.part_in + ((size_t)t2 * a.s_in * a.Bm + b) * 32 + 4 * g;
                    for (int cc = 0; cc < a.s_in; ++cc, p += (size_t)a.Bm * 32) {
                        acc0 += ldf4(p);
                        acc1 += ldf4(p + 16);
                    }
                }
            }
        }
        if (finish) {
            if (kind == 0) {
                const int e = 32 * t2 + 4 * g;
                if (valid) {
                    f32x4 s0v, s1v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        s0v[i] = sigmoidf_(acc0[i]);
                        s1v[i] = sigmoidf_(acc1[i]);
                    }
                    const f32x4 b0 = a.bias ? ldf4(a.bias + e) : zero4();
                    const f32x4 b1 = a.bias ? ldf4(a.bias + e + 16) : zero4();
                    float *sr = a.score + (size_t)b * a.E + e;
                    float *kr = a.key + (size_t)b * a.E + e;
                    stf4(sr, s0v);
                    stf4(sr + 16, s1v);
                    stf4(kr, s0v + b0);
                    stf4(kr + 16, s1v + b1);
                }
                if (wave_arrive(&a.gctr[G_ROUTER_DONE]) == (uint32_t)a.router_target - 1u) {
                    topk_loop(a, s_mask);
                    continue;
                }
            } else if (kind == 1) {
                const int l = 32 * (t2 - a.n_r2) + 4 * g;
                if (valid) {
                    const size_t o = (size_t)b * a.L + l;
                    store_hl4(a.z_hi + o, a.z_lo + o, acc0);
                    store_hl4(a.z_hi + o + 16, a.z_lo + o + 16, acc1);
                }
            } else {
                const int i0 = 16 * (t2 - a.n_r2 - n_l2) + 4 * g;
                if (valid) {
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = silu_mul(acc0[i], acc1[i]);
                    const size_t o = (size_t)b * a.Is + i0;
                    store_hl4(a.ash_hi + o, a.ash_lo + o, v);
                }
            }
        }
        if (a.router_target > 0 && a.n_r2 > 0) maybe_join_topk(a, s_mask);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: expert gate/up (MXFP4) + SwiGLU.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void swiglu_store(const StepArgs &a, int p, int row0, f32x4 vg,
                                             f32x4 vu) {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = silu_mul(vg[i], vu[i]);
    const size_t o = (size_t)p * a.I + row0;
    store_hl4(a.act_hi + o, a.act_lo + o, v);
}

template <int SPC>
__global__ void __launch_bounds__(kBlock) k_w13(const StepArgs a) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int NC = a.meta[M_N_COLS];
    const int PT = a.I >> 4;
    const int total = NC * PT * a.s13;
    const int nwaves = gridDim.x * kWavesPerBlock;
    const size_t qrow = a.L / 2, srow = a.L / 32;
    for (int u = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); u < total; u += nwaves) {
        const int c = u % a.s13, r = u / a.s13, pt = r % PT, cu = r / PT;
        const int e = a.cu_expert[cu], p0 = a.cu_p0[cu], nt = a.cu_n[cu];
        const int s0 = c * SPC;
        const size_t rg = (size_t)e * 2 * a.I + 16 * pt + n, ru = rg + a.I;
        const bool valid = col < nt;
        const int p = p0 + col;
        const int tok = valid ? a.pair_slot[p] / a.k : 0;
        const uint16_t *X = (part ? a.z_lo : a.z_hi) + (size_t)tok * a.L + 32 * g;
        f32x4 accg = zero4(), accu = zero4();
        fp4_chunk<SPC>(a.w13_q + rg * qrow + 16 * g, a.w13_s + rg * srow,
                       a.w13_q + ru * qrow + 16 * g, a.w13_s + ru * srow, X, valid, g, s0, accg,
                       accu);
        accg = add_pair_column(accg);
        accu = add_pair_column(accu);
        const bool writer = valid && part == 0;
        if (a.s13 == 1) {
            if (writer) swiglu_store(a, p, 16 * pt + 4 * g, accg, accu);
            continue;
        }
        float *mine = a.part13 + (((size_t)p * PT + pt) * a.s13 + c) * 32 + 4 * g;
        if (writer) {
            stf4(mine, accg);
            stf4(mine + 16, accu);
        }
        uint32_t *ctr = a.ctr13 + (size_t)cu * PT + pt;
        if (wave_arrive(ctr) != (uint32_t)(a.s13 - 1)) continue;
        acquire_agent();
        wave_store_counter(ctr, 0u);
        if (writer) {
            const float *q = a.part13 + ((size_t)p * PT + pt) * a.s13 * 32 + 4 * g;
            f32x4 vg = zero4(), vu = zero4();
            for (int cc = 0; cc < a.s13; ++cc, q += 32) {
                vg += ldf4(q);
                vu += ldf4(q + 16);
            }
            swiglu_store(a, p, 16 * pt + 4 * g, vg, vu);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 3: expert down (MXFP4) + weighted combine in latent space.
// ---------------------------------------------------------------------------

// ylat for rows [r0, r0+32) of every token: sum over the token's experts in
// ascending id of w * (sum of the K-chunk partials in chunk order).
__device__ __noinline__ void combine_latent_tile(const StepArgs &a, int r0) {
    const int lane = lane_id();
    for (int it = lane; it < a.B * 8; it += kWave) {
        const int b = it >> 3, q = it & 7;
        f32x4 acc = zero4();
        for (int j = 0; j < a.k; ++j) {
            const int slot = b * a.k + j;
            const int p = a.pair_of_slot[slot];
            const float w = a.wsel[slot];
            const float *src = a.ypart + (size_t)p * a.s2 * a.L + r0 + 4 * q;
            f32x4 t = zero4();
            for (int cc = 0; cc < a.s2; ++cc, src += a.L) t += ldf4(src);
            acc += w * t;
        }
        const size_t o = (size_t)b * a.L + r0 + 4 * q;
        store_hl4(a.ylat_hi + o, a.ylat_lo + o, acc);
    }
}

template <int SPC>
__global__ void __launch_bounds__(kBlock) k_w2(const StepArgs a) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int NC = a.meta[M_N_COLS];
    const int LT = a.L >> 5;
    const int total = NC * LT * a.s2;
    const int nwaves = gridDim.x * kWavesPerBlock;
    const size_t qrow = a.I / 2, srow = a.I / 32;
    const uint32_t target = (uint32_t)(NC * a.s2);
    for (int u = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); u < total; u += nwaves) {
        const int c = u % a.s2, r = u / a.s2, lt = r % LT, cu = r / LT;
        const int e = a.cu_expert[cu], p0 = a.cu_p0[cu], nt = a.cu_n[cu];
        const int s0 = c * SPC;
        const size_t r0 = (size_t)e * a.L + 32 * lt + n, r1 = r0 + 16;
        const bool valid = col < nt;
        const int p = p0 + (valid ? col : 0);
        const uint16_t *X = (part ? a.act_lo : a.act_hi) + (size_t)p * a.I + 32 * g;
        f32x4 acc0 = zero4(), acc1 = zero4();
        fp4_chunk<SPC>(a.w2_q + r0 * qrow + 16 * g, a.w2_s + r0 * srow,
                       a.w2_q + r1 * qrow + 16 * g, a.w2_s + r1 * srow, X, valid, g, s0, acc0,
                       acc1);
        acc0 = add_pair_column(acc0);
        acc1 = add_pair_column(acc1);
        if (valid && part == 0) {
            float *mine = a.ypart + ((size_t)p * a.s2 + c) * a.L + 32 * lt + 4 * g;
            stf4(mine, acc0);
            stf4(mine + 16, acc1);
        }
        uint32_t *ctr = a.ctr2 + lt;
        if (wave_arrive(ctr) != target - 1u) continue;
        acquire_agent();
        wave_store_counter(ctr, 0u);
        combine_latent_tile(a, 32 * lt);
    }
}

// ---------------------------------------------------------------------------
// Kernel 4: latent-up + shared-down, bf16 output.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void store_out4(uint16_t *dst, f32x4 v) {
    *(u32x2 *)dst = (u32x2){bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                            bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
}

template <int SPC>
__global__ void __launch_bounds__(kBlock) k_out(const StepArgs a) {
    // The routing counters of the dense input kernel are cleared here, where
    // no wave of the step can touch them any more.
    if (blockIdx.x == 0 && threadIdx.x < 3) a.gctr[threadIdx.x] = 0u;
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const int col = n >> 1, part = n & 1;
    const int ncg = (a.B + 7) >> 3;
    const int n_t2 = a.H >> 5;
    const int total = n_t2 * ncg * a.s_out;
    const int nwaves = gridDim.x * kWavesPerBlock;
    for (int u = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); u < total; u += nwaves) {
        const int c = u % a.s_out, r = u / a.s_out, cg = r % ncg, t2 = r / ncg;
        const int s0 = c * SPC;
        const int b = 8 * cg + col;
        const bool valid = b < a.B;
        const int bb = valid ? b : 0;
        const size_t h0 = 32 * (size_t)t2 + n;
        TwoSource t;
        t.A0a = a.lat_up + h0 * a.L + 32 * g;
        t.A1a = t.A0a + (size_t)16 * a.L;
        t.Xa = (part ? a.ylat_lo : a.ylat_hi) + (size_t)bb * a.L + 32 * g;
        t.A0b = a.sh_w2 + h0 * a.Is + 32 * g;
        t.A1b = t.A0b + (size_t)16 * a.Is;
        t.Xb = (part ? a.ash_lo : a.ash_hi) + (size_t)bb * a.Is + 32 * g;
        t.Ls = a.L / kKStep;
        f32x4 acc0 = zero4(), acc1 = zero4();
        out_chunk<SPC>(t, valid, s0, acc0, acc1);
        acc0 = add_pair_column(acc0);
        acc1 = add_pair_column(acc1);
        const bool writer = valid && part == 0;
        if (a.s_out > 1) {
            float *mine = a.part_out + ((size_t)(t2 * a.s_out + c) * a.Bm + bb) * 32 + 4 * g;
            if (writer) {
                stf4(mine, acc0);
                stf4(mine + 16, acc1);
            }
            uint32_t *ctr = a.ctr_out + t2 * a.ncg_out_cap + cg;
            if (wave_arrive(ctr) != (uint32_t)(a.s_out - 1)) continue;
            acquire_agent();
            wave_store_counter(ctr, 0u);
            if (!writer) continue;
            acc0 = zero4();
            acc1 = zero4();
            const float *p = a.part_out + ((size_t)t2 * a.s_out * a.Bm + bb) * 32 + 4 * g;
            for (int cc = 0; cc < a.s_out; ++cc, p += (size_t)a.Bm * 32) {
                acc0 += ldf4(p);
                acc1 += ldf4(p + 16);
            }
        }
        if (writer) {
            uint16_t *o = a.out + (size_t)b * a.H + 32 * t2 + 4 * g;
            store_out4(o, acc0);
            store_out4(o + 16, acc1);
        }
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

__device__ __forceinline__ float hl_val(const uint16_t *hi, const uint16_t *lo, size_t i) {
    return bf16_val(hi[i]) + bf16_val(lo[i]);
}

__global__ void k_debug_export(const StepArgs a, const DebugArgs d) {
    const size_t tid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t nE = (size_t)a.B * a.E, nL = (size_t)a.B * a.L, nS = (size_t)a.B * a.Is;
    const size_t nA = (size_t)a.B * a.k * a.I;
    for (size_t i = tid; i < nE; i += stride) {
        if (d.score) d.score[i] = a.score[i];
        if (d.key) d.key[i] = a.key[i];
    }
    for (size_t i = tid; i < nL; i += stride) {
        if (d.z) d.z[i] = hl_val(a.z_hi, a.z_lo, i);
        if (d.ylat) d.ylat[i] = hl_val(a.ylat_hi, a.ylat_lo, i);
    }
    for (size_t i = tid; i < nS; i += stride)
        if (d.ash) d.ash[i] = hl_val(a.ash_hi, a.ash_lo, i);
    for (size_t i = tid; i < nA; i += stride) {
        if (!d.act) break;
        const size_t slot = i / a.I, col = i % a.I;
        const size_t p = (size_t)a.pair_of_slot[slot];
        d.act[i] = hl_val(a.act_hi, a.act_lo, p * a.I + col);
    }
    if (tid == 0 && d.n_active) d.n_active[0] = a.meta[M_N_ACTIVE];
}

}  // namespace moe
