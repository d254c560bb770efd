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
    // Launch plan.
    int32_t n_r2;             // 32-row router tiles computed by the dense input kernel
    int32_t router_target;    // arrivals on G_ROUTER_DONE that complete the router
    int32_t s_in, spc_in;     // K splits / steps per split: router + latent-down + shared gate/up
    int32_t s_out, spc_out;   // latent-up + shared-down
    int32_t s13, spc13;       // expert gate/up
    int32_t s2, spc2;         // expert down
    int32_t ncg_in_cap, ncg_out_cap;  // column-group strides of the dense counters
    int32_t ncols_cap;        // capacity of the expert column-unit list
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
    uint32_t *gctr, *ctr_in, *ctr_out, *ctr13, *ctr2;
    int32_t *meta;
    float *score, *key;
    int32_t *idx;
    float *wsel;
    int32_t *act_expert, *act_off, *cu_expert, *cu_p0, *cu_n, *pair_slot, *pair_of_slot;
    uint16_t *z_hi, *z_lo, *ash_hi, *ash_lo, *act_hi, *act_lo, *ylat_hi, *ylat_lo;
    float *part_in, *part_out, *part13, *ypart;
};

}  // namespace moe
