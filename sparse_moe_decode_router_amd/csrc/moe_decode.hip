// moe_decode.hip - host side of the decode-step library: configuration checks,
// workspace carving, the batch-dependent launch plan and the C ABI declared in
// include/moe_decode.h.  The kernels live in kernels.h.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "moe_decode.h"
#include "plan.h"

using namespace moe;
using namespace moe::plan;

namespace {

typedef void (*StepKernel)(const StepArgs);

// Fused step kernels, one per (gate/up chunk, down chunk) pair of the shapes
// the library is built for; other shapes run the four-launch step.
struct FusedEntry {
    int s13, s2;
    StepKernel k;
};
const FusedEntry kFused[] = {{16, 16, k_step<16, 16>}, {16, 8, k_step<16, 8>},
                             {16, 4, k_step<16, 4>},   {16, 2, k_step<16, 2>},
                             {8, 8, k_step<8, 8>},     {4, 3, k_step<4, 3>},
                             {2, 2, k_step<2, 2>}};

// Second launch of the two-launch step, for the same chunk shapes.
const FusedEntry kTail[] = {{16, 16, k_tail<16, 16>}, {16, 8, k_tail<16, 8>},
                            {16, 4, k_tail<16, 4>},   {16, 2, k_tail<16, 2>},
                            {8, 8, k_tail<8, 8>},     {4, 3, k_tail<4, 3>},
                            {2, 2, k_tail<2, 2>}};

StepKernel tail_kernel(const moe_decode_config &c, const Plan &p) {
    if (c.router_dtype != MOE_ROUTER_BF16 || p.sd.kw == 0 || p.lu.kw == 0) return nullptr;
    for (const FusedEntry &f : kTail)
        if (f.s13 == p.s13 && f.s2 == p.s2) return f.k;
    return nullptr;
}

StepKernel fused_kernel(const moe_decode_config &c, const Plan &p) {
    if (c.router_dtype != MOE_ROUTER_BF16 || p.sd.kw == 0 || p.lu.kw == 0) return nullptr;
    for (const FusedEntry &f : kFused)
        if (f.s13 == p.s13 && f.s2 == p.s2) return f.k;
    return nullptr;
}

#define MOE_SPC_TABLE(K)                                                                      \
    {nullptr, K<1>, K<2>,  K<3>,  K<4>,  K<5>,  K<6>,  K<7>, K<8>,                                \
     K<9>,    K<10>, K<11>, K<12>, K<13>, K<14>, K<15>, K<16>}
#define MOE_W13_TABLE(L)                                                                       \
    {nullptr,        k_w13<1, L>,  k_w13<2, L>,  k_w13<3, L>,  k_w13<4, L>,  k_w13<5, L>,        \
     k_w13<6, L>,    k_w13<7, L>,  k_w13<8, L>,  k_w13<9, L>,  k_w13<10, L>, k_w13<11, L>,       \
     k_w13<12, L>,   k_w13<13, L>, k_w13<14, L>, k_w13<15, L>, k_w13<16, L>}
const StepKernel kW13[] = MOE_W13_TABLE(false);
// Gate/up kernels that run the routing first (batches up to 8).
const StepKernel kW13Late[] = MOE_W13_TABLE(true);
// Gate/up kernels with KS waves per tile (chunk shapes 2, 4, 8 and 16).
struct W13Split {
    int s, ks;
    StepKernel k, k_late;
};
const W13Split kW13Split[] = {
    {2, 2, k_w13<2, false, 2>, k_w13<2, true, 2>},    {4, 2, k_w13<4, false, 2>, k_w13<4, true, 2>},
    {4, 4, k_w13<4, false, 4>, k_w13<4, true, 4>},    {8, 2, k_w13<8, false, 2>, k_w13<8, true, 2>},
    {8, 4, k_w13<8, false, 4>, k_w13<8, true, 4>},    {8, 8, k_w13<8, false, 8>, k_w13<8, true, 8>},
    {16, 2, k_w13<16, false, 2>, k_w13<16, true, 2>}, {16, 4, k_w13<16, false, 4>, k_w13<16, true, 4>},
    {16, 8, k_w13<16, false, 8>, k_w13<16, true, 8>}};

StepKernel w13_kernel(int s, int ks, bool late) {
    if (ks == 1) return late ? kW13Late[s] : kW13[s];
    for (const W13Split &w : kW13Split)
        if (w.s == s && w.ks == ks) return late ? w.k_late : w.k;
    return nullptr;
}
#undef MOE_W13_TABLE
#undef MOE_SPC_TABLE
#define MOE_W2_TABLE(KS)                                                                       \
    {nullptr,        k_w2<1, KS>,  k_w2<2, KS>,  k_w2<3, KS>,  k_w2<4, KS>,  k_w2<5, KS>,        \
     k_w2<6, KS>,    k_w2<7, KS>,  k_w2<8, KS>,  k_w2<9, KS>,  k_w2<10, KS>, k_w2<11, KS>,       \
     k_w2<12, KS>,   k_w2<13, KS>, k_w2<14, KS>, k_w2<15, KS>, k_w2<16, KS>}
const StepKernel kW2[] = MOE_W2_TABLE(1);
#undef MOE_W2_TABLE
#define MOE_W2_TABLE(KS)                                                                       \
    {nullptr,              k_w2<1, KS, true>,  k_w2<2, KS, true>,  k_w2<3, KS, true>,          \
     k_w2<4, KS, true>,    k_w2<5, KS, true>,  k_w2<6, KS, true>,  k_w2<7, KS, true>,          \
     k_w2<8, KS, true>,    k_w2<9, KS, true>,  k_w2<10, KS, true>, k_w2<11, KS, true>,         \
     k_w2<12, KS, true>,   k_w2<13, KS, true>, k_w2<14, KS, true>, k_w2<15, KS, true>,         \
     k_w2<16, KS, true>}
// Down kernels of the ordered latent combine.
const StepKernel kW2Ord[] = MOE_W2_TABLE(1);
#undef MOE_W2_TABLE
// Down kernels with two waves per tile (even chunk shapes only).
const StepKernel kW2Split[] = {nullptr,        nullptr,       k_w2<2, 2>,  nullptr,
                               k_w2<4, 2>,     nullptr,       k_w2<6, 2>,  nullptr,
                               k_w2<8, 2>,     nullptr,       k_w2<10, 2>, nullptr,
                               k_w2<12, 2>,    nullptr,       k_w2<14, 2>, nullptr,
                               k_w2<16, 2>};
const StepKernel kW2SplitOrd[] = {nullptr,              nullptr,             k_w2<2, 2, true>,
                                  nullptr,              k_w2<4, 2, true>,    nullptr,
                                  k_w2<6, 2, true>,     nullptr,             k_w2<8, 2, true>,
                                  nullptr,              k_w2<10, 2, true>,   nullptr,
                                  k_w2<12, 2, true>,    nullptr,             k_w2<14, 2, true>,
                                  nullptr,              k_w2<16, 2, true>};

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

struct moe_decode_ctx {
    moe_decode_config cfg;
    moe_decode_weights w;
    char *ws;
    size_t ws_bytes;
    Layout lay;
    int device;
    int32_t last_hip;
    moe_decode_dispatch_info last;
    hipEvent_t events[14];  // timing events (caller-owned), n_events = 0: off
    int32_t n_events;
    int32_t mode;           // MOE_MODE_*
    // Side-stream step: the library's second stream (default priority) and
    // the fork / join events between it and the caller's stream.
    hipStream_t side;
    hipEvent_t fork_ev, join_ev;
    // Layer whose router and latent-down rows the dense-in launch prefetches
    // (moe_decode_set_next_layer; NULL: none).
    const moe_decode_ctx *next;
    int32_t n_cus;          // compute units of the device
    StepKernel occ_kernel;  // fused kernel whose occupancy is cached
    int32_t occ_blocks;     // its resident workgroups per compute unit
};

struct moe_decode_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace {

moe_status hip_fail(moe_decode_ctx *ctx, hipError_t e) {
    if (ctx) ctx->last_hip = (int32_t)e;
    return MOE_ERR_HIP;
}

StepArgs base_args(const moe_decode_ctx *ctx) {
    const moe_decode_config &c = ctx->cfg;
    const Layout &l = ctx->lay;
    char *ws = ctx->ws;
    StepArgs a;
    std::memset(&a, 0, sizeof a);
    a.H = c.hidden;
    a.L = c.latent;
    a.E = c.n_experts;
    a.I = c.expert_inter;
    a.Is = c.shared_inter;
    a.Bm = c.max_batch;
    a.km = c.max_top_k;
    a.ncols_cap = ncols_cap(c.n_experts, c.max_batch, c.max_top_k);
    const moe_decode_weights &w = ctx->w;
    if (c.router_dtype == MOE_ROUTER_BF16)
        a.router_w = (const uint16_t *)w.router_w;
    else
        a.router_w32 = (const float *)w.router_w;
    a.bias = w.router_bias;
    a.lat_down = w.lat_down;
    a.lat_up = w.lat_up;
    a.w13_q = w.w13_q;
    a.w13_s = w.w13_s;
    a.w2_q = w.w2_q;
    a.w2_s = w.w2_s;
    a.sh_w13 = w.sh_w13;
    a.sh_w2 = w.sh_w2;
    a.gctr = (uint32_t *)(ws + l.gctr);
    a.meta = (int32_t *)(ws + l.meta);
    a.score = (float *)(ws + l.score);
    a.key = (float *)(ws + l.key);
    a.idx = (int32_t *)(ws + l.idx);
    a.wsel = (float *)(ws + l.wsel);
    a.act_expert = (int32_t *)(ws + l.act_expert);
    a.act_off = (int32_t *)(ws + l.act_off);
    a.cu_rec = (int32_t *)(ws + l.cu_rec);
    a.pair_slot = (int32_t *)(ws + l.pair_slot);
    a.pair_of_slot = (int32_t *)(ws + l.pair_of_slot);
    a.zhl = (uint16_t *)(ws + l.zhl);
    a.ashhl = (uint16_t *)(ws + l.ashhl);
    a.acthl = (uint16_t *)(ws + l.acthl);
    a.ylat = (float *)(ws + l.ylat);
    a.ysh = (float *)(ws + l.ysh);
    a.pout = (float *)(ws + l.pout);
    a.cctr = (uint32_t *)(ws + l.cctr);
    a.c13 = (uint32_t *)(ws + l.c13);
    a.part = (float *)(ws + l.part);
    a.rpart = (float *)(ws + l.rpart);
    a.rgc = (uint32_t *)(ws + l.rgc);
    a.kx_tiles = dense_tiles(ctx->cfg);
    a.kx_groups = cdiv(a.kx_tiles, kWG);
    return a;
}

int grid_for(long long units, long long cap_blocks) {
    return (int)std::max(1LL, std::min(units, cap_blocks));
}

}  // namespace

extern "C" {

moe_status moe_decode_validate_config(const moe_decode_config *c) {
    return plan::validate_config(c);
}

size_t moe_decode_workspace_size(const moe_decode_config *c) {
    if (moe_decode_validate_config(c) != MOE_OK) return 0;
    return make_layout(*c).total;
}

const char *moe_decode_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or device";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    }
    return "unknown status";
}

int32_t moe_decode_last_hip_error(const moe_decode_ctx *ctx) { return ctx ? ctx->last_hip : 0; }

moe_status moe_decode_init(const moe_decode_config *cfg, const moe_decode_weights *w,
                           void *workspace, size_t workspace_bytes, moe_decode_ctx **out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    moe_status st = moe_decode_validate_config(cfg);
    if (st != MOE_OK) return st;
    if (!w) return MOE_ERR_INVALID_ARG;
    const void *req[] = {w->router_w, w->lat_down, w->lat_up, w->w13_q, w->w13_s,
                         w->w2_q,     w->w2_s,     w->sh_w13, w->sh_w2};
    for (const void *p : req)
        if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
    if (w->router_bias && !aligned16(w->router_bias)) return MOE_ERR_INVALID_ARG;
    const Layout lay = make_layout(*cfg);
    if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) || workspace_bytes < lay.total)
        return MOE_ERR_WORKSPACE;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return MOE_ERR_HIP;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_UNSUPPORTED;

    moe_decode_ctx *ctx = new (std::nothrow) moe_decode_ctx();
    if (!ctx) return MOE_ERR_HIP;
    ctx->cfg = *cfg;
    ctx->w = *w;
    ctx->ws = (char *)workspace;
    ctx->ws_bytes = workspace_bytes;
    ctx->lay = lay;
    ctx->device = dev;
    ctx->last_hip = 0;
    ctx->n_events = 0;
    ctx->mode = MOE_MODE_FOUR_LAUNCHES;
    ctx->n_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    ctx->occ_kernel = nullptr;
    ctx->occ_blocks = 1;
    ctx->side = nullptr;
    ctx->fork_ev = ctx->join_ev = nullptr;
    ctx->next = nullptr;
    std::memset(&ctx->last, 0, sizeof ctx->last);
    e = hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ctx->fork_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ctx->join_ev, hipEventDisableTiming);
    if (e != hipSuccess) {
        moe_decode_destroy(ctx);
        return MOE_ERR_HIP;
    }

    // Every counter starts at zero; the step returns them to zero itself.
    const size_t nwords = lay.counters_end / 4;
    hipLaunchKernelGGL(k_fill_u32, dim3(std::min<size_t>(1024, (nwords + 255) / 256)), dim3(256),
                       0, nullptr, (uint32_t *)ctx->ws, nwords, 0u);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) {
        moe_decode_destroy(ctx);
        return MOE_ERR_HIP;
    }
    *out = ctx;
    return MOE_OK;
}

moe_status moe_decode_step(moe_decode_ctx *ctx, const uint16_t *x, int32_t batch, int32_t top_k,
                           uint16_t *out, int32_t *topk_idx, float *topk_w, moe_stream_t stream) {
    if (!ctx || !x || !out) return MOE_ERR_INVALID_ARG;
    const moe_decode_config &c = ctx->cfg;
    if (batch < 1 || batch > c.max_batch || top_k < 1 || top_k > c.max_top_k)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || ((uintptr_t)out & 7u) || ((uintptr_t)topk_idx & 3u) ||
        ((uintptr_t)topk_w & 3u))
        return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    Plan pl = make_plan(c, batch, top_k, ctx->mode == MOE_MODE_FUSED);
    const StepKernel fused = ctx->mode == MOE_MODE_FUSED ? fused_kernel(c, pl) : nullptr;
    if (!fused) pl = make_plan(c, batch, top_k, false);
    const StepKernel tail = ctx->mode == MOE_MODE_TWO_LAUNCHES ? tail_kernel(c, pl) : nullptr;
    const bool side = ctx->mode == MOE_MODE_SIDE_STREAM && pl.sd.kw > 0 && pl.lu.kw > 0;
    // The routing at the start of the gate/up launch instead of at the end of
    // the dense-in launch (up to 8 tokens and kLatePairs pairs; not with a
    // next-layer prefetch, whose units wait for the router in dense-in).
    // Gate/up kernel of the multi-launch forms: when its units would fill less
    // than the two resident workgroups per compute unit, KS waves share each
    // tile (KS in {2, 4, 8}, the smallest that fills them, where a kernel of
    // that shape exists).
    int ks13 = 1;
    if (!fused && !tail) {
        const long long cols = ncols_cap(c.n_experts, batch, top_k);
        for (int ks = 2; ks <= kWG && cols * pl.tg13 * ks13 < 2LL * ctx->n_cus; ks *= 2) {
            if (!w13_kernel(pl.s13, ks, false)) break;
            ks13 = ks;
        }
        pl.units_13 = cols * cdiv(c.expert_inter / 8, kWG / ks13);
    }
    const long long cap = 65528;  // workgroups (a multiple of the XCD count); more units loop
    // The late gate/up launch is persistent: one workgroup per resident slot
    // (two per compute unit), each routing once and running up to
    // kLateUnitsPerWG units.
    const long long late_grid = std::min<long long>(pl.units_13, 2LL * ctx->n_cus);
    // Where the routing runs.  MOE_MODE_LATE_ROUTING: at the start of the
    // gate/up launch wherever that form applies; MOE_MODE_DENSE_ROUTING:
    // always in the dense-in launch; the default (MOE_MODE_FOUR_LAUNCHES and
    // the side-stream form): late when the dense-in launch runs in one round
    // of resident workgroups, where the routing at its end would be a tail
    // with the memory idle (a launch of more rounds hides it under its last
    // round, and the gate/up workgroups would only pay for it again).
    // 9 to 16 tokens in a dense-in launch of one round of resident
    // workgroups (the TP8 share): the K-sliced dense-in kernel, whose router
    // slices finish early and whose routing units overlap the other row
    // groups' stream, where the routing after a one-round launch is a tail
    // (TP8 share batch 16: 91.2 -> 87.6 us; K3, 1.4 rounds, stays: 208 -> 212
    // at batch 9).
    const bool kx_small = !fused && !tail && !side && batch > kWG && pl.ncg_in == 1 &&
                          c.router_dtype == MOE_ROUTER_BF16 && pl.units_in <= 2LL * ctx->n_cus;
    const bool late_ok = c.router_dtype == MOE_ROUTER_BF16 && batch <= kWG &&
                         batch * top_k <= kLatePairs && !ctx->next &&
                         pl.units_13 <= (long long)kLateUnitsPerWG * late_grid;
    const bool dense_one_round = pl.units_in <= 2LL * ctx->n_cus;
    const bool late = late_ok && (ctx->mode == MOE_MODE_LATE_ROUTING ||
                                  ((ctx->mode == MOE_MODE_FOUR_LAUNCHES ||
                                    ctx->mode == MOE_MODE_SIDE_STREAM ||
                                    ctx->mode == MOE_MODE_ORDERED) && dense_one_round));
    StepArgs a = base_args(ctx);
    a.B = batch;
    a.k = top_k;
    a.x = x;
    a.out = out;
    a.user_idx = topk_idx;
    a.user_w = topk_w;
    a.n_rtiles = pl.n_rtiles;
    // Arrivals that complete the router: one per router unit of the dense
    // input kernel, or one per workgroup of the f32 router kernel.
    a.router_target = c.router_dtype == MOE_ROUTER_BF16 ? pl.n_rtiles * (fused ? pl.ncg_in : 1)
                                                        : cdiv(c.n_experts, kWavesPerBlock);
    a.kw_in = pl.in.kw;
    a.kw_out = pl.out.kw;
    a.out_rows = pl.out_rows;
    a.router_rows = pl.router_rows;
    a.latent_rows = pl.latent_rows;
    a.spc_in = pl.in.spc;
    a.spc_out = pl.out.spc;
    const int n_main = pl.n_rtiles + c.latent / pl.latent_rows;  // router + latent-down tiles
    a.dense_lo = 0;
    a.dense_hi = n_main + c.shared_inter / 8;
    a.zero_ylat = 1;
    // Above 8 tokens the routing is spread over routing units (8 tokens
    // each) appended to the dense-in launch.
    a.route_units = c.router_dtype == MOE_ROUTER_BF16 && batch > 8 ? cdiv(batch, kWG) : 0;
    a.pf_units = 0;
    if (ctx->next) {
        const moe_decode_config &nc = ctx->next->cfg;
        a.pf0 = (const uint8_t *)ctx->next->w.router_w;
        a.pf_bytes0 = (uint64_t)nc.n_experts * nc.hidden *
                      (nc.router_dtype == MOE_ROUTER_F32 ? 4 : 2);
        a.pf1 = (const uint8_t *)ctx->next->w.lat_down;
        a.pf_bytes1 = (uint64_t)nc.latent * nc.hidden * 2;
        a.pf_units = (int32_t)((a.pf_bytes0 + a.pf_bytes1 + kPfUnit - 1) / kPfUnit);
    }

    moe_decode_dispatch_info &d = ctx->last;
    d.batch = batch;
    d.top_k = top_k;
    d.col_tiles = pl.ncg_in;
    d.split_in = pl.in.kw;
    d.split_out = pl.out.kw;
    d.split_w13 = ks13;
    // Expert chunks: from 2 tokens the gate/up kernel, and above 8 the down
    // kernel, take 8 of the 16 steps per chunk where that would be 16 (K
    // split 1): half the LDS, three resident workgroups instead of two (K3
    // batch 2 / 8 / 64 step: 103.5 / 199.0 / 515.6 -> 100.3 / 192.3 / 493.3
    // us; the down kernel from 2 tokens lost 1-2 us).
    const int s13 = batch > 1 && ks13 == 1 && pl.s13 == 16 ? 8 : pl.s13;
    const int s2_one = batch > 8 && pl.s2 == 16 ? 8 : pl.s2;
    // Four-launch down kernel: when its units would fill less than the two
    // resident workgroups per compute unit, two waves share each tile (twice
    // the units, half the steps per wave).
    const bool split2 = !fused && !tail && pl.s2 % 2 == 0 && pl.units_2 < 2LL * ctx->n_cus;
    if (split2) pl.units_2 = (long long)ncols_cap(c.n_experts, batch, top_k) *
                             cdiv(c.latent / 16, kWG / 2);
    d.split_w2 = split2 ? 2 : 1;
    // The latent combine in a fixed order (MOE_MODE_ORDERED).
    const bool ordered = ctx->mode == MOE_MODE_ORDERED;
    d.ordered = ordered ? 1 : 0;
    const StepKernel w2_k = ordered ? (split2 ? kW2SplitOrd[pl.s2] : kW2Ord[pl.s2])
                                    : (split2 ? kW2Split[pl.s2] : kW2[s2_one]);
    d.grid_in = (int32_t)(pl.units_in + a.route_units);  // every unit its own workgroup
    // Expert grids for the expected column units (ncols_grid); the kernels
    // loop over the rest.
    const long long cols_all = ncols_cap(c.n_experts, batch, top_k);
    const long long cols_grid = ncols_grid(c.n_experts, batch, top_k);
    d.grid_w13 = late ? (int32_t)late_grid : grid_for(pl.units_13 / cols_all * cols_grid, cap);
    d.grid_w2 = grid_for(pl.units_2 / cols_all * cols_grid, cap);
    d.grid_out = grid_for(pl.units_out, cap);
    d.router_f32 = c.router_dtype == MOE_ROUTER_F32;
    d.fused = fused ? 1 : tail ? 2 : side ? 3 : 0;
    d.routing = d.router_f32 ? 3 : late ? 2 : a.route_units ? 1 : 0;
    d.n_kernels = fused ? 1 : tail ? 2 : side ? 6 + d.router_f32 : 4 + d.router_f32;
    d.grid_step = 0;
    d.out_staged = 0;
    d.in_staged = 0;
    // One persistent workgroup per resident slot of `kernel` (the unit
    // queues do not rely on residency; this only sizes the grid).
    auto persistent_grid = [&](StepKernel kernel, long long units) {
        if (ctx->occ_kernel != kernel) {
            int blocks = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kWGThreads, 0) !=
                    hipSuccess ||
                blocks < 1)
                blocks = 1;
            ctx->occ_kernel = kernel;
            ctx->occ_blocks = blocks;
        }
        return (int32_t)std::max(1LL, std::min<long long>(units, (long long)ctx->occ_blocks *
                                                                     ctx->n_cus));
    };
    if (tail) {
        a.kw_sd = pl.sd.kw;
        a.spc_sd = pl.sd.spc;
        a.kw_lu = pl.lu.kw;
        a.spc_lu = pl.lu.spc;
        a.tg13 = pl.tg13;
        a.tg2 = pl.tg2;
        const int n_ot = cdiv(c.hidden, pl.out_rows);
        a.n_sd_units = cdiv(n_ot, kWG / pl.sd.kw) * pl.ncg_out;
        a.n_lu_units = cdiv(n_ot, kWG / pl.lu.kw) * pl.ncg_out;
        a.n_sd_first = a.n_sd_units / 2;
        d.grid_step = persistent_grid(tail, pl.units_13 + pl.units_2 + a.n_sd_units +
                                                a.n_lu_units);
    }
    if (fused) {
        a.u_lat = pl.u_lat;
        a.u_sh = pl.u_sh;
        a.u_13 = pl.u_13;
        a.u_sd = pl.u_sd;
        a.u_2 = pl.u_2;
        a.u_lu = pl.u_lu;
        a.u_end = pl.u_end;
        a.kw_sd = pl.sd.kw;
        a.spc_sd = pl.sd.spc;
        a.kw_lu = pl.lu.kw;
        a.spc_lu = pl.lu.spc;
        a.tg13 = pl.tg13;
        a.tg2 = pl.tg2;
        a.n_lat_units = pl.u_sh - pl.u_lat;
        a.n_sh_units = pl.u_13 - pl.u_sh;
        a.n_sd_units = pl.u_lu - pl.u_sd;
        d.grid_step = persistent_grid(fused, pl.u_end);
    }

    const bool timed = ctx->n_events == 2 * d.n_kernels;
    int ki = 0;
    auto launch_on = [&](hipStream_t st, StepKernel kernel, unsigned grid, unsigned threads,
                         const StepArgs &args, size_t lds = 0) {
        if (timed)
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, st, ctx->events[2 * ki],
                                  ctx->events[2 * ki + 1], 0, args);
        else
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, st, args);
        ++ki;
    };
    auto launch = [&](StepKernel kernel, unsigned grid, unsigned threads) {
        launch_on(s, kernel, grid, threads, a);
    };
    if (fused) {
        launch(fused, d.grid_step, kWGThreads);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e);
    }
    const StepKernel dense_in[] = {late ? k_dense_in<1, false> : k_dense_in<1, true>,
                                   k_dense_in<2, true>, k_dense_in<3, true>, k_dense_in<4, true>};
    const StepKernel dense_in_kx[] = {k_dense_in_kx<1>, k_dense_in_kx<2>, k_dense_in_kx<3>,
                                      k_dense_in_kx<4>};
    // Above 16 tokens (and kx_small) the dense-in launch stages x in LDS per
    // row group of 8 tiles and splits K into slices, about two units per
    // compute unit.
    const bool kx = (pl.ncg_in >= 2 || kx_small) && pl.latent_rows == 16 && pl.router_rows == 16;
    // Up to 2 tokens: x staged in LDS, six weight steps in flight per wave
    // (K3 batch 1: 32.0 -> 28.5 us).  3 to 8 tokens, where the launch fits
    // one workgroup per compute unit: all 8 rows staged, once per compute
    // unit (TP8 share batch 3 / 4 / 8: -0.3 / -0.4 / -0.9 us per layer; K3,
    // whose 696 tiles would re-stage them 2.7 times per compute unit, keeps
    // the unstaged kernel: batch 3-5 +1 us with it).
    const bool xl_wide = batch > kXlTokens && pl.units_in <= ctx->n_cus;
    const bool xl = !fused && (batch <= kXlTokens || (batch <= kXlTokensWide && xl_wide)) &&
                    pl.in.spc >= kXlRing && pl.in.spc <= kMaxStepsPerChunk &&
                    c.hidden <= kMaxDenseK && a.route_units == 0;
    d.in_staged = kx ? 2 : xl && xl_wide ? 3 : xl ? 1 : 0;
    auto dense_launch = [&](hipStream_t st, StepArgs &args) {
        if (xl) {
            const int rw_in = kWG / pl.in.kw;
            launch_on(st,
                      xl_wide ? (late ? k_dense_in_xl8<false> : k_dense_in_xl8<true>)
                              : (late ? k_dense_in_xl<false> : k_dense_in_xl<true>),
                      (unsigned)(dense_units_host(args.dense_hi - args.dense_lo, rw_in, 1) +
                                 args.route_units + args.pf_units),
                      kWGThreads, args);
            return;
        }
        if (!kx) {
            const int rw_in = kWG / pl.in.kw;
            launch_on(st, dense_in[pl.ncg_in - 1],
                      (unsigned)(dense_units_host(args.dense_hi - args.dense_lo, rw_in, 1) +
                                 args.route_units + args.pf_units),
                      kWGThreads, args);
            return;
        }
        // Router row groups (when this launch holds the router) in the
        // shortest slices; the other row groups in as many slices as the
        // compute units' remaining workgroup slots (two per unit) hold.
        const int nsteps = c.hidden / kKStep;
        const int nrg = cdiv(args.dense_hi - args.dense_lo, kWG);
        args.kx_rg_r = args.dense_lo == 0 && pl.n_rtiles > 0 ? std::min(nrg, cdiv(pl.n_rtiles, kWG)) : 0;
        const int nrg_o = nrg - args.kx_rg_r;
        auto slices_o = [&](int units_r, int route) {
            const int slots = 2 * ctx->n_cus - units_r - route - args.pf_units;
            return nrg_o > 0 ? std::max(1, std::min({kMaxSlices, nsteps, slots / nrg_o})) : 1;
        };
        int sps_r = cdiv(nsteps, std::min(kMaxSlices, nsteps));
        if (args.kx_rg_r > 0) {
            // The routing units add the router's slices (kRouteTokensTp
            // tokens each, one round trip): more of them than with keys in
            // memory.  The router slices lengthen until the other row groups
            // keep the slice count they would have next to cdiv(B, 8)
            // routing units; the router counter counts router slices.
            const int want = slices_o(args.kx_rg_r * cdiv(nsteps, sps_r), args.route_units);
            args.route_units = cdiv(batch, kRouteTokensTp);
            while (sps_r < nsteps && slices_o(args.kx_rg_r * cdiv(nsteps, sps_r), args.route_units) < want)
                ++sps_r;
            args.router_target = args.kx_rg_r * cdiv(nsteps, sps_r);
        }
        args.kx_sps_r = sps_r;
        const int units_r = args.kx_rg_r * cdiv(nsteps, args.kx_sps_r);
        int nsl = slices_o(units_r, args.route_units);
        args.kx_sps = cdiv(nsteps, nsl);
        nsl = cdiv(nsteps, args.kx_sps);
        launch_on(st, dense_in_kx[pl.ncg_in - 1],
                  (unsigned)(units_r + nrg_o * nsl + args.route_units + args.pf_units), kWGThreads, args);
    };
    if (side) {
        // The shared expert depends on x alone: its gate/up and down launches
        // run on the side stream while the routed path runs on the caller's;
        // the latent-up launch joins them.
        a.kw_sd = pl.sd.kw;
        a.spc_sd = pl.sd.spc;
        a.kw_lu = pl.lu.kw;
        a.spc_lu = pl.lu.spc;
        const int n_ot = cdiv(c.hidden, pl.out_rows);
        StepArgs sa = a;
        a.dense_hi = n_main;
        sa.dense_lo = n_main;
        sa.zero_ylat = 0;
        sa.route_units = 0;
        sa.pf_units = 0;
        hipError_t e = hipEventRecord(ctx->fork_ev, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(ctx->side, ctx->fork_ev, 0);
        if (e != hipSuccess) return hip_fail(ctx, e);
        if (d.router_f32) launch(k_router_f32, cdiv(c.n_experts, kWavesPerBlock), kBlock);
        dense_launch(s, a);
        dense_launch(ctx->side, sa);
        launch(w13_kernel(s13, ks13, late), d.grid_w13, kWGThreads);
        launch(w2_k, d.grid_w2, kWGThreads);
        launch_on(ctx->side, k_out_part<OUT_SHARED>,
                  grid_for(dense_units_host(n_ot, kWG / pl.sd.kw, pl.ncg_out), cap), kWGThreads,
                  sa);
        e = hipEventRecord(ctx->join_ev, ctx->side);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, ctx->join_ev, 0);
        if (e != hipSuccess) return hip_fail(ctx, e);
        launch(k_out_part<OUT_LATENT>,
               grid_for(dense_units_host(n_ot, kWG / pl.lu.kw, pl.ncg_out), cap), kWGThreads);
        e = hipGetLastError();
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e);
    }
    if (d.router_f32) launch(k_router_f32, cdiv(c.n_experts, kWavesPerBlock), kBlock);
    dense_launch(s, a);
    if (tail) {
        launch(tail, d.grid_step, kWGThreads);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e);
    }
    launch(w13_kernel(s13, ks13, late), d.grid_w13, kWGThreads);
    launch(w2_k, d.grid_w2, kWGThreads);
    if (pl.ncg_out >= 2) {
        // Above 8 tokens: the column operands staged in LDS per group of 8
        // output tiles, K in slices (about two units per compute unit).
        const int n_ot = cdiv(c.hidden, pl.out_rows), nrg = cdiv(n_ot, kWG);
        const int nsteps = (c.latent + c.shared_inter) / kKStep;
        int nsl = std::max(1, std::min({kMaxSlicesOut, nsteps, (2 * ctx->n_cus + nrg / 2) / nrg}));
        a.kx_sps_out = cdiv(nsteps, nsl);
        nsl = cdiv(nsteps, a.kx_sps_out);
        const StepKernel out_kx = pl.ncg_out <= 2 ? k_out_kx<2> : pl.ncg_out <= 4 ? k_out_kx<4>
                                                                                    : k_out_kx<8>;
        launch(out_kx, (unsigned)(nrg * nsl + 2 * nrg), kWGThreads);  // slice units, then sum units
    } else {
        // Up to two tokens the column operands of the whole reduction fit in
        // LDS, up to eight their ylat part: staged once per workgroup.
        const size_t st_full = (size_t)4 * batch * (c.latent + c.shared_inter);
        const size_t st_lat = (size_t)4 * batch * c.latent;
        const bool one_unit = pl.out.kw > 0 && d.grid_out == (int32_t)pl.units_out;
        if (one_unit && batch <= kOutStTokens && st_full <= (size_t)kOutStBytes) {
            launch_on(s, k_out_st<true>, d.grid_out, kWGThreads, a, st_full);
            d.out_staged = 1;
        } else if (one_unit && batch <= kOutStLatTokens && st_lat <= (size_t)kOutStLatBytes) {
            launch_on(s, k_out_st<false>, d.grid_out, kWGThreads, a, st_lat);
            d.out_staged = 2;
        } else {
            const StepKernel out_k[] = {k_out<1>, k_out<2>, k_out<3>, k_out<4>};
            launch(out_k[pl.ncg_unit_out - 1], d.grid_out, kWGThreads);
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(ctx, e);
    return MOE_OK;
}

moe_status moe_decode_destroy(moe_decode_ctx *ctx) {
    if (!ctx) return MOE_ERR_INVALID_ARG;
    if (ctx->side) (void)hipStreamDestroy(ctx->side);
    if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
    if (ctx->join_ev) (void)hipEventDestroy(ctx->join_ev);
    delete ctx;
    return MOE_OK;
}

moe_status moe_decode_graph_create(moe_decode_ctx *const *ctxs, int32_t n_layers,
                                   const uint16_t *const *x, int32_t batch, int32_t top_k,
                                   uint16_t *const *out, int32_t *const *topk_idx,
                                   float *const *topk_w, moe_decode_graph **graph) {
    if (!ctxs || n_layers < 1 || !x || !out || !graph) return MOE_ERR_INVALID_ARG;
    *graph = nullptr;
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_ctx *c = ctxs[i];
        if (!c || !x[i] || !out[i] || batch < 1 || batch > c->cfg.max_batch || top_k < 1 ||
            top_k > c->cfg.max_top_k)
            return MOE_ERR_INVALID_ARG;
    }
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(ctxs[0], e);
    moe_status st = MOE_OK;
    hipGraph_t g = nullptr;
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        for (int i = 0; i < n_layers && st == MOE_OK; ++i)
            st = moe_decode_step(ctxs[i], x[i], batch, top_k, out[i],
                                 topk_idx ? topk_idx[i] : nullptr, topk_w ? topk_w[i] : nullptr,
                                 (moe_stream_t)cs);
        const hipError_t e2 = hipStreamEndCapture(cs, &g);
        if (e == hipSuccess) e = e2;
    }
    hipGraphExec_t ex = nullptr;
    if (e == hipSuccess && st == MOE_OK) e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cs);
    if (st != MOE_OK || e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return st != MOE_OK ? st : hip_fail(ctxs[0], e);
    }
    moe_decode_graph *gr = new (std::nothrow) moe_decode_graph();
    if (!gr) {
        (void)hipGraphExecDestroy(ex);
        (void)hipGraphDestroy(g);
        return MOE_ERR_HIP;
    }
    gr->graph = g;
    gr->exec = ex;
    *graph = gr;
    return MOE_OK;
}

moe_status moe_decode_graph_launch(moe_decode_graph *graph, moe_stream_t stream) {
    if (!graph) return MOE_ERR_INVALID_ARG;
    return hipGraphLaunch(graph->exec, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_decode_graph_destroy(moe_decode_graph *graph) {
    if (!graph) return MOE_ERR_INVALID_ARG;
    (void)hipGraphExecDestroy(graph->exec);
    (void)hipGraphDestroy(graph->graph);
    delete graph;
    return MOE_OK;
}

moe_status moe_decode_last_dispatch(const moe_decode_ctx *ctx, moe_decode_dispatch_info *info) {
    if (!ctx || !info) return MOE_ERR_INVALID_ARG;
    *info = ctx->last;
    return MOE_OK;
}

moe_status moe_decode_set_timing_events(moe_decode_ctx *ctx, void *const *events, int32_t n) {
    if (!ctx || n < 0) return MOE_ERR_INVALID_ARG;
    const int32_t want = 2 * (4 + (ctx->cfg.router_dtype == MOE_ROUTER_F32 ? 1 : 0));
    if (n == 0) {
        ctx->n_events = 0;
        return MOE_OK;
    }
    const int32_t want_side = want + 4;  // six (seven with the f32 router) launches
    if ((n != want && n != want_side && n != 2 && n != 4) || !events) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) {
        if (!events[i]) return MOE_ERR_INVALID_ARG;
        ctx->events[i] = (hipEvent_t)events[i];
    }
    ctx->n_events = n;
    return MOE_OK;
}

moe_status moe_decode_set_next_layer(moe_decode_ctx *ctx, const moe_decode_ctx *next) {
    if (!ctx || next == ctx) return MOE_ERR_INVALID_ARG;
    ctx->next = next;
    return MOE_OK;
}

moe_status moe_decode_set_mode(moe_decode_ctx *ctx, int32_t mode) {
    if (!ctx || (mode != MOE_MODE_FUSED && mode != MOE_MODE_FOUR_LAUNCHES &&
                 mode != MOE_MODE_TWO_LAUNCHES && mode != MOE_MODE_SIDE_STREAM &&
                 mode != MOE_MODE_LATE_ROUTING && mode != MOE_MODE_DENSE_ROUTING &&
                 mode != MOE_MODE_ORDERED))
        return MOE_ERR_INVALID_ARG;
    ctx->mode = mode;
    return MOE_OK;
}

moe_status moe_decode_read_flags(moe_decode_ctx *ctx, uint32_t *flags) {
    if (!ctx || !flags) return MOE_ERR_INVALID_ARG;
    const hipError_t e = hipMemcpy(flags, ctx->ws + ctx->lay.gctr + 4 * G_ERROR, 4,
                                   hipMemcpyDeviceToHost);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e);
}

moe_status moe_decode_debug_export(moe_decode_ctx *ctx, int32_t batch, int32_t top_k,
                                   const moe_decode_debug *dbg, moe_stream_t stream) {
    if (!ctx || !dbg || batch < 1 || batch > ctx->cfg.max_batch || top_k < 1 ||
        top_k > ctx->cfg.max_top_k)
        return MOE_ERR_INVALID_ARG;
    StepArgs a = base_args(ctx);
    a.B = batch;
    a.k = top_k;
    const DebugArgs d{dbg->score, dbg->key, dbg->z, dbg->act, dbg->ylat, dbg->ash, dbg->n_active};
    hipLaunchKernelGGL(k_debug_export, dim3(256), dim3(256), 0, (hipStream_t)stream, a, d);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e);
}

moe_status moe_decode_debug_dequant(const uint8_t *q, const uint8_t *s, int64_t n, float *out,
                                    moe_stream_t stream) {
    if (!q || !s || !out || n <= 0 || n % 32 || ((uintptr_t)q & 3u)) return MOE_ERR_INVALID_ARG;
    const int64_t threads = n / 8;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, q, s, n, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The step without a caller workspace
// ---------------------------------------------------------------------------

namespace {

// The workspace of moe_decode_step_static: one static array per device, held
// by the loaded code object until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is taken
// once per device with hipGetSymbolAddress and used from then on.
static __device__ __align__(256) unsigned char scratch[MOE_DECODE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;

struct StaticDevice {
    std::once_flag once;
    hipError_t err = hipSuccess;
    bool gfx950 = false;
    int n_cus = 1;
    char *ptr = nullptr;  // device address of `scratch` on this device
};
StaticDevice g_static[kMaxDevices];

}  // namespace

extern "C" moe_status moe_decode_step_static(const moe_decode_config *cfg,
                                             const moe_decode_weights *w, const uint16_t *x,
                                             int32_t batch, int32_t top_k, uint16_t *out,
                                             int32_t *topk_idx, float *topk_w,
                                             moe_stream_t stream) {
    moe_status st = plan::validate_config(cfg);
    if (st != MOE_OK) return st;
    if (!w) return MOE_ERR_INVALID_ARG;
    const void *req[] = {w->router_w, w->lat_down, w->lat_up, w->w13_q, w->w13_s,
                         w->w2_q,     w->w2_s,     w->sh_w13, w->sh_w2};
    for (const void *p : req)
        if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
    if (w->router_bias && !aligned16(w->router_bias)) return MOE_ERR_INVALID_ARG;
    const Layout lay = make_layout(*cfg);
    if (lay.total > (size_t)MOE_DECODE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    StaticDevice &sd = g_static[dev];
    std::call_once(sd.once, [&sd, dev]() {
        hipDeviceProp_t prop;
        sd.err = hipGetDeviceProperties(&prop, dev);
        if (sd.err != hipSuccess) return;
        sd.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        sd.n_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
        if (sd.gfx950) sd.err = hipGetSymbolAddress((void **)&sd.ptr, HIP_SYMBOL(scratch));
    });
    if (sd.err != hipSuccess) return MOE_ERR_HIP;
    if (!sd.gfx950) return MOE_ERR_UNSUPPORTED;
    if (!sd.ptr) return MOE_ERR_HIP;
    // A context on the stack over the static array, in the four-launch form.
    moe_decode_ctx ctx{};
    ctx.cfg = *cfg;
    ctx.w = *w;
    ctx.ws = sd.ptr;
    ctx.ws_bytes = MOE_DECODE_STATIC_WORKSPACE_BYTES;
    ctx.lay = lay;
    ctx.device = dev;
    ctx.mode = MOE_MODE_FOUR_LAUNCHES;
    ctx.n_cus = sd.n_cus;
    ctx.occ_blocks = 1;
    // The array keeps what the last call left: the counters start at zero
    // (a fill kernel, not a memset, so that the call stays capturable).
    const size_t nwords = lay.counters_end / 4;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)std::min<size_t>(1024, (nwords + 255) / 256)),
                       dim3(256), 0, (hipStream_t)stream, (uint32_t *)sd.ptr, nwords, 0u);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    return moe_decode_step(&ctx, x, batch, top_k, out, topk_idx, topk_w, stream);
}
