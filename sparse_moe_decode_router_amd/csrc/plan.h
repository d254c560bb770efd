// plan.h - host-side planning of the decode step: configuration checks, the
// batch-dependent launch plan (K splits, unit counts) and the carving of the
// caller's workspace.  Plain C++ (no HIP headers), shared by the library and
// by a host-only test build under the address and undefined-behaviour
// sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "moe_limits.h"
#include "moe_decode.h"

namespace moe {
namespace plan {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// K split of one kernel: KW waves of a workgroup share the K range of a row
// group, each taking SPC consecutive 128-element steps (KW * SPC = K / 128,
// KW in {8, 4, 2, 1}, SPC <= kMaxStepsPerChunk); the largest KW is chosen.
struct Split {
    int kw, spc;
};

inline Split choose_split(int nsteps) {
    for (int kw = kWG; kw >= 1; kw /= 2)
        if (nsteps % kw == 0 && nsteps / kw <= kMaxStepsPerChunk) return Split{kw, nsteps / kw};
    return Split{0, 0};
}

// Column units of the expert kernels: at most min(E, B k) experts are active,
// each split into units of <= 8 tokens (B k pairs give at most B k / 8 extra
// units).
inline int ncols_cap(int E, int B, int k) { return std::min(E, B * k) + cdiv(B * k, 8); }

// Column units to size the expert launches for: the distinct experts that
// B k uniformly spread selections would touch, E (1 - (1 - 1/E)^(B k)), plus
// 10 %, at most the capacity.  The kernels loop over units with the grid
// stride, so more units are still all processed; fewer leave fewer
// workgroups that only read the unit count and exit (at 64 tokens on the
// K3 layer the capacity is 1,024 units against about 620 used).
inline int ncols_grid(int E, int B, int k) {
    const double e = E, pk = (double)B * k;
    const double d = e * (1.0 - std::pow(1.0 - 1.0 / e, pk));
    return std::min(ncols_cap(E, B, k), (int)std::ceil(1.1 * d) + 1);
}

// Steps per staged chunk of the expert kernels: the largest divisor of
// K / 128 that is at most 16.
inline int expert_chunk(int nsteps) {
    for (int s = 16; s >= 1; --s)
        if (nsteps % s == 0) return s;
    return 1;
}

// Rows per output tile: 16, unless that gives more tiles than the 256
// compute units of MI355X take at once; then the hidden rows are split into
// 2 x 256 tiles (two workgroups per compute unit) of at most 16 rows, so that
// every unit gets the same share.
inline int out_tile_rows(int H) {
    if (cdiv(H, 16) <= 256) return 16;
    return std::min(16, cdiv(H, 2 * 256));
}

// Unit count of a dense kernel (tile groups padded to a multiple of the XCD
// count, times the column groups); matches dense_units() in the kernels.
inline long long dense_units_host(int n_t, int RW, int ncg) {
    return (long long)cdiv(cdiv(n_t, RW), kXcds) * kXcds * ncg;
}

struct Plan {
    int n_rtiles, ncg_in, ncg_out, ncg_unit_out, out_rows;
    Split in, out, sd, lu;
    int s13, s2, tg13, tg2;
    long long units_in, units_out, units_13, units_2;
    // Fused step: unit ranges (see StepArgs).
    int u_lat, u_sh, u_13, u_2, u_sd, u_lu, u_end;
    int router_rows, latent_rows;
};

// Rows of the router and latent-down tiles: short in the fused step (the
// router and z finish early, so the routing and the expert units start
// sooner), 16 in the four-launch step (fewer units).
constexpr int kFusedRouterRows = 4, kFusedLatentRows = 8;

inline Plan make_plan(const moe_decode_config &c, int B, int k, bool fused) {
    Plan p;
    p.router_rows = fused ? kFusedRouterRows : 16;
    p.latent_rows = fused ? kFusedLatentRows : 16;
    p.n_rtiles = c.router_dtype == MOE_ROUTER_BF16 ? c.n_experts / p.router_rows : 0;
    p.ncg_in = cdiv(B, 16);
    p.ncg_out = cdiv(B, 8);
    p.in = choose_split(c.hidden / kKStep);
    p.out = choose_split((c.latent + c.shared_inter) / kKStep);
    p.s13 = expert_chunk(c.latent / kKStep);
    p.s2 = expert_chunk(c.expert_inter / kKStep);
    // Dense-in tiles: router, latent-down, then shared tiles of 8 gate + 8 up
    // rows.
    const int n_t_in = p.n_rtiles + c.latent / p.latent_rows + c.shared_inter / 8;
    const long long cols = ncols_cap(c.n_experts, B, k);
    // Four-launch dense-in units cover every column group; the fused step's
    // take one group each.
    p.units_in = dense_units_host(n_t_in, kWG / p.in.kw, fused ? p.ncg_in : 1);
    p.out_rows = out_tile_rows(c.hidden);
    // Output units: NCG column groups of 8 tokens each (at most 4, whose f32
    // operand loads still fit the registers), every tile once per block.
    p.ncg_unit_out = p.ncg_out <= 4 ? p.ncg_out : cdiv(p.ncg_out, 2);
    p.units_out = dense_units_host(cdiv(c.hidden, p.out_rows), kWG / p.out.kw,
                                   cdiv(p.ncg_out, p.ncg_unit_out));
    // Expert kernels: 8 row tiles per workgroup (8 gate + 8 up rows, or 16
    // latent rows, per tile).
    p.tg13 = cdiv(c.expert_inter / 8, kWG);
    p.tg2 = cdiv(c.latent / 16, kWG);
    p.units_13 = cols * p.tg13;
    p.units_2 = cols * p.tg2;
    // Fused step: the output units split into shared-down (K = Is) and
    // latent-up (K = L) units; every range holds whole tile groups of one
    // kind for each column group.
    p.sd = choose_split(c.shared_inter / kKStep);
    p.lu = choose_split(c.latent / kKStep);
    const int rw_in = kWG / std::max(1, p.in.kw);
    const int n_ot = cdiv(c.hidden, p.out_rows);
    p.u_lat = cdiv(p.n_rtiles, rw_in) * p.ncg_in;
    p.u_sh = p.u_lat + cdiv(c.latent / p.latent_rows, rw_in) * p.ncg_in;
    p.u_13 = p.u_sh + cdiv(c.shared_inter / 8, rw_in) * p.ncg_in;
    p.u_2 = p.u_13 + (int)p.units_13;
    p.u_sd = p.u_2 + (int)p.units_2;
    p.u_lu = p.u_sd + cdiv(n_ot, kWG / std::max(1, p.sd.kw)) * p.ncg_out;
    p.u_end = p.u_lu + cdiv(n_ot, kWG / std::max(1, p.lu.kw)) * p.ncg_out;
    return p;
}

// Dense-in tiles of the four-launch plan (16-row router and latent tiles,
// shared tiles of 8 gate + 8 up rows) and their row groups of 8.
inline int dense_tiles(const moe_decode_config &c) {
    return (c.router_dtype == MOE_ROUTER_BF16 ? c.n_experts / 16 : 0) + c.latent / 16 +
           c.shared_inter / 8;
}
constexpr int kMaxGroupsOut = 8;   // column groups of 8 tokens per output unit

// The counter area has one size for every configuration, so that contexts of
// different configurations can share a workspace: the per-column-unit
// counters for the largest possible column-unit list, and the per-row-group
// counters of the large-batch kernels for the largest row-group count (dense
// tiles of kMaxExperts router rows, a latent and a shared size below
// kMaxDenseK; output tiles of a hidden size up to kMaxDenseK).
constexpr int kMaxCols = kMaxExperts + kMaxBatch * kMaxTopK / 8;
constexpr int kMaxRowGroups = (kMaxExperts / 16 + kMaxDenseK / 16 + kMaxDenseK / 8 + kWG - 1) / kWG;
static_assert(kMaxCols >= kMaxExperts && kMaxRowGroups >= kMaxDenseK / 16 / kWG, "limits");

struct Layout {
    size_t gctr, meta, c13, rgc, cctr, score, key, idx, wsel, act_expert, act_off, cu_rec,
        pair_slot, pair_of_slot, zhl, ashhl, acthl, ylat, ysh, pout, part, rpart, total;
    size_t counters_end;  // [0, counters_end) holds every counter: cleared at init
};

// Row groups of 8 tiles the large-batch kernels keep a counter for.
inline int row_groups(const moe_decode_config &c) {
    const int n_ot = cdiv(c.hidden, out_tile_rows(c.hidden));
    return std::max(cdiv(dense_tiles(c), kWG), cdiv(n_ot, kWG));
}

// Bytes of the counter area (the same for every configuration).
inline size_t counter_bytes() {
    size_t o = 0;
    o = align_up(o + G_COUNT * 4);
    o = align_up(o + M_COUNT * 4);
    o = align_up(o + (size_t)kMaxCols * kCtrStride * 4);
    o = align_up(o + (size_t)2 * kMaxRowGroups * kCtrStride * 4);
    o = align_up(o + (size_t)kMaxBatch * kOrdGroups * kOrdStride * 4);
    return o;
}

inline Layout make_layout(const moe_decode_config &c) {
    const size_t Bm = c.max_batch, km = c.max_top_k, E = c.n_experts, L = c.latent,
                 I = c.expert_inter, Is = c.shared_inter;
    const size_t P = Bm * km;
    const size_t ncols = (size_t)ncols_cap((int)E, (int)Bm, (int)km);
    Layout l;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    // Counters, at fixed offsets for every configuration.
    l.gctr = take(G_COUNT * 4);
    l.meta = take(M_COUNT * 4);
    l.c13 = take((size_t)kMaxCols * kCtrStride * 4);
    l.rgc = take((size_t)2 * kMaxRowGroups * kCtrStride * 4);  // caller's and side stream's launches
    l.cctr = take((size_t)kMaxBatch * kOrdGroups * kOrdStride * 4);  // ordered latent combine
    l.counters_end = o;
    // Score and key rows are padded to kMaxExperts: the routing reads a whole
    // row with one base address (entries past E are never used).
    l.score = take(Bm * kMaxExperts * 4);
    l.key = take(Bm * kMaxExperts * 4);
    l.idx = take(P * 4);
    l.wsel = take(P * 4);
    l.act_expert = take((std::min(E, P) + 1) * 4);
    l.act_off = take((std::min(E, P) + 1) * 4);
    l.cu_rec = take(ncols * kRecWords * 4);
    l.pair_slot = take(P * 4);
    l.pair_of_slot = take(P * 4);
    l.zhl = take(Bm * 2 * L * 2);
    l.ashhl = take(Bm * 2 * Is * 2);
    l.acthl = take(P * 2 * I * 2);
    l.ylat = take(Bm * L * 4);
    l.ysh = take(Bm * (size_t)c.hidden * 4);
    // Slice partials of the large-batch dense-in (above 16 tokens) and output
    // (above 8 tokens) kernels, and the pair outputs of the ordered latent
    // combine (down launch, between those two): no two of them are live at
    // the same time (the ordered combine has no side stream).
    const size_t n_ot = (size_t)cdiv(c.hidden, out_tile_rows(c.hidden));
    const size_t ncg = (size_t)cdiv(c.max_batch, 16);
    // K-sliced dense-in partials: above 16 tokens, and from 9 where that kernel
    // also serves (a dense-in launch of one round).
    const size_t part_in = c.max_batch > kWG ? (size_t)kMaxSlices * dense_tiles(c) * ncg * kWave * 16 : 0;
    // The output kernel's column groups per unit: 2, 4 or 8 (ceil(B / 8) rounded up).
    const size_t gout = c.max_batch <= 16 ? 2 : c.max_batch <= 32 ? 4 : kMaxGroupsOut;
    const size_t part_out = c.max_batch > 8 ? kMaxSlicesOut * n_ot * gout * kWave * 16 : 0;
    // The router's K-slice partials of that dense-in kernel, token-major
    // ([slice][token][kMaxExperts] f32, read by the routing units), after its
    // other partials.
    const size_t rpart = part_in ? (size_t)kMaxSlices * Bm * kMaxExperts * 4 : 0;
    l.part = take(std::max({part_in + rpart, part_out, P * L * 4}));
    l.rpart = l.part + part_in;
    l.pout = l.part;
    l.total = o;
    return l;
}

// The checks of moe_decode_validate_config.
inline moe_status validate_config(const moe_decode_config *c) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->hidden <= 0 || c->latent <= 0 || c->n_experts <= 0 || c->expert_inter <= 0 ||
        c->shared_inter <= 0 || c->max_batch <= 0 || c->max_top_k <= 0)
        return MOE_ERR_INVALID_ARG;
    if (c->router_dtype != MOE_ROUTER_BF16 && c->router_dtype != MOE_ROUTER_F32)
        return MOE_ERR_INVALID_ARG;
    if (c->max_top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
    if (c->max_batch > kMaxBatch || c->max_top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (c->hidden % kKStep || c->latent % kKStep || c->expert_inter % kKStep ||
        c->shared_inter % kKStep)
        return MOE_ERR_UNSUPPORTED;
    if (c->n_experts % 32 || c->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    // The dense reduction lengths must split into KW x SPC steps (see
    // choose_split); the expert kernels take any multiple of 128.
    const int ks[2] = {c->hidden, c->latent + c->shared_inter};
    for (int K : ks)
        if (choose_split(K / kKStep).kw == 0) return MOE_ERR_UNSUPPORTED;
    // Offsets are formed in 32-bit ints where they index one token or pair,
    // and byte offsets into the shared gate/up matrix (2 Is rows of H bf16)
    // in 32 bits.
    if ((long long)c->hidden * c->shared_inter > (1LL << 29) ||
        (long long)c->n_experts * 2 * c->expert_inter > (1LL << 31))
        return MOE_ERR_UNSUPPORTED;
    if (row_groups(*c) > kMaxRowGroups) return MOE_ERR_UNSUPPORTED;  // implied by the above
    return MOE_OK;
}

}  // namespace plan
}  // namespace moe
