// step_args.h - the argument block every decode-step kernel receives by value:
// layer dimensions, the batch-dependent launch plan, weight / input / output
// pointers and the carved workspace.
#pragma once

#include <stdint.h>

namespace moe {

struct StepArgs {
    // Layer and step dimensions.
    int32_t H, L, E, I, Is;   // hidden, latent, experts, expert inter., shared inter.
    int32_t B, k;             // tokens and experts per token of this step
    int32_t Bm, km;           // capacities (context max_batch / max_top_k)
    // Launch plan: waves of a workgroup that split K in each kernel (the
    // rest of the 8 waves take further row groups).
    int32_t n_rtiles;         // router tiles (router_rows rows each) of the dense-in units
    int32_t router_target;    // arrivals on G_ROUTER_DONE that complete the router
    int32_t kw_in, kw_out;
    int32_t spc_in, spc_out;  // 128-element steps per wave in the dense kernels
    int32_t ncols_cap;        // capacity of the expert column-unit list
    int32_t out_rows;         // rows per output tile (<= 16)
    // Fused step: unit ranges [0, u_lat) router, [u_lat, u_sh) latent-down,
    // [u_sh, u_13) shared gate/up, [u_13, u_2) gate/up, [u_2, u_sd) down,
    // [u_sd, u_lu) shared-down, [u_lu, u_end) latent-up; K splits of the two
    // output kinds; tile groups per column unit; unit counts waited for.
    int32_t u_lat, u_sh, u_13, u_2, u_sd, u_lu, u_end;
    int32_t router_rows, latent_rows;  // valid rows of router / latent-down tiles (<= 16)
    int32_t kw_sd, spc_sd, kw_lu, spc_lu;
    int32_t tg13, tg2;
    int32_t n_lat_units, n_sh_units, n_sd_units;
    // Two-launch step (dense-in, then one persistent launch): shared-down
    // units placed before the down units, latent-up units.
    int32_t n_sd_first, n_lu_units;
    // Dense-in launch: tiles [dense_lo, dense_hi) of the list [router |
    // latent-down | shared gate/up]; zero_ylat: this launch clears ylat.
    int32_t dense_lo, dense_hi, zero_ylat;
    // Routing units appended to the dense-in launch (0: the workgroup that
    // completes the router routes the whole step).
    int32_t route_units;
    // Dense-in above 16 tokens: steps per K slice, tiles and row groups of
    // the whole tile list (partial-buffer stride and counter offset).
    int32_t kx_sps, kx_tiles, kx_groups;
    // ... row groups [0, kx_rg_r) (those holding router tiles) take shorter
    // slices of kx_sps_r steps, so that the router completes early.
    int32_t kx_rg_r, kx_sps_r;
    int32_t kx_sps_out;  // output kernel above 8 tokens: steps per K slice
    // Prefetch units of the dense-in launch (0: none): a following layer's
    // rows [pf0, pf0 + pf_bytes0) and [pf1, pf1 + pf_bytes1).
    int32_t pf_units;
    const uint8_t *pf0, *pf1;
    uint64_t pf_bytes0, pf_bytes1;
    // Weights (borrowed).
    const uint16_t *router_w;
    const float *router_w32;
    const float *bias;
    const uint16_t *lat_down, *lat_up;
    const uint8_t *w13_q, *w13_s, *w2_q, *w2_s;
    const uint16_t *sh_w13, *sh_w2;
    // Step input / outputs.
    const uint16_t *x;
    uint16_t *out;
    int32_t *user_idx;
    float *user_w;
    // Workspace.
    uint32_t *gctr;
    uint32_t *c13;  // fused step: gate/up units done per column unit [ncols_cap], 256 B apart
    int32_t *meta;
    float *score, *key;
    int32_t *idx;
    float *wsel;
    int32_t *act_expert, *act_off, *cu_rec, *pair_slot, *pair_of_slot;
    // Intermediates as bf16 hi/lo row pairs: zhl [B][2][L], acthl [pair][2][I],
    // ashhl [B][2][Is] (row 0: hi = bf16(v), row 1: lo = bf16(v - hi)).
    uint16_t *zhl, *acthl, *ashhl;
    float *ylat;  // f32 latent combine (atomic adds)
    float *ysh;   // fused step: shared-down sums [B][H] f32
    // Ordered latent combine: each pair's weighted down output [pair][L] f32
    // (pairs in token order, b k + j) and the arrivals per (token, tile group).
    float *pout;
    uint32_t *cctr;
    float *part;    // dense-in above 16 tokens: slice partials [slice][tile][group][lane][4]
    float *rpart;   // ... the router tiles' partials [slice][token][kMaxExperts]
    uint32_t *rgc;  // ... arrivals per row group, 256 B apart (two sets: caller / side stream)
};

}  // namespace moe
