// plan_check.cpp - host-only check of the library's planning code (plan.h)
// under the address and undefined-behaviour sanitizers: configuration
// validation, workspace carving and launch plans over the configurations the
// tests and the benchmark use and a seeded sweep of random ones, valid and
// invalid.  Exits non-zero (or the sanitizer aborts) on the first violation.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "plan.h"

using namespace moe;
using namespace moe::plan;

static int failures = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);    \
            if (++failures > 20) std::exit(1);                                        \
        }                                                                             \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {  // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int pick(const std::vector<int> &v) { return v[next_u32() % v.size()]; }

static void check_layout(const moe_decode_config &c) {
    const Layout l = make_layout(c);
    CHECK(l.counters_end == counter_bytes());
    CHECK(l.gctr == 0);
    const size_t regions[] = {l.gctr, l.meta, l.c13, l.rgc, l.score, l.key, l.idx, l.wsel,
                              l.act_expert, l.act_off, l.cu_rec, l.pair_slot, l.pair_of_slot,
                              l.zhl, l.ashhl, l.acthl, l.ylat, l.ysh, l.part};
    size_t prev = 0;
    for (size_t i = 0; i < sizeof regions / sizeof regions[0]; ++i) {
        CHECK(regions[i] % kAlign == 0);
        CHECK(i == 0 || regions[i] > prev);
        CHECK(regions[i] <= l.total);
        prev = regions[i];
    }
    CHECK(l.score >= l.counters_end);
    // Sizes the kernels rely on.
    const size_t Bm = c.max_batch, km = c.max_top_k;
    CHECK(l.key - l.score >= Bm * kMaxExperts * 4);
    CHECK(l.cu_rec + (size_t)ncols_cap(c.n_experts, c.max_batch, c.max_top_k) * kRecWords * 4 <=
          l.pair_slot);
    CHECK(l.ylat - l.acthl >= Bm * km * 2 * (size_t)c.expert_inter * 2);
    CHECK(l.total - l.ysh >= Bm * (size_t)c.hidden * 4);
    CHECK(row_groups(c) <= kMaxRowGroups);
    CHECK(ncols_cap(c.n_experts, c.max_batch, c.max_top_k) <= kMaxCols);
}

static void check_plans(const moe_decode_config &c) {
    const int bs[] = {1, 2, 3, 7, 8, 9, 16, 17, 32, 33, 63, 64};
    for (int B : bs) {
        if (B > c.max_batch) continue;
        for (int k = 1; k <= c.max_top_k; k += (k < 4 ? 1 : 5)) {
            for (int fused = 0; fused < 2; ++fused) {
                const Plan p = make_plan(c, B, k, fused != 0);
                CHECK(p.in.kw > 0 && p.out.kw > 0);
                CHECK(p.in.kw * p.in.spc * kKStep == c.hidden);
                CHECK(p.out.kw * p.out.spc * kKStep == c.latent + c.shared_inter);
                CHECK(p.units_in > 0 && p.units_out > 0 && p.units_13 > 0 && p.units_2 > 0);
                CHECK(p.s13 >= 1 && p.s13 <= 16 && (c.latent / kKStep) % p.s13 == 0);
                CHECK(p.s2 >= 1 && p.s2 <= 16 && (c.expert_inter / kKStep) % p.s2 == 0);
                CHECK(p.out_rows >= 1 && p.out_rows <= 16);
                CHECK(p.ncg_in == (B + 15) / 16 && p.ncg_out == (B + 7) / 8);
                CHECK(p.u_lat <= p.u_sh && p.u_sh <= p.u_13 && p.u_13 <= p.u_2 &&
                      p.u_2 <= p.u_sd && p.u_sd <= p.u_lu && p.u_lu <= p.u_end);
                CHECK(ncols_cap(c.n_experts, B, k) <= kMaxCols);
            }
        }
    }
}

int main() {
    // The layers of the tests and the benchmark.
    const moe_decode_config named[] = {
        {7168, 2048, 896, 2048, 4096, 64, 16, MOE_ROUTER_BF16},  // K3 layer
        {7168, 2048, 896, 256, 512, 64, 16, MOE_ROUTER_BF16},    // one TP8 rank's share
        {512, 256, 64, 256, 512, 1, 4, MOE_ROUTER_F32},          // 64-expert layer
        {1024, 512, 96, 384, 384, 64, 8, MOE_ROUTER_BF16},       // small test layer
        {256, 256, 64, 256, 256, 64, 4, MOE_ROUTER_BF16},
        {8192, 4096, 1024, 8192, 4096, 64, 64, MOE_ROUTER_BF16}, // the largest shapes
    };
    for (const moe_decode_config &c : named) {
        CHECK(validate_config(&c) == MOE_OK);
        check_layout(c);
        check_plans(c);
    }
    // Invalid configurations are refused.
    moe_decode_config bad = named[0];
    bad.max_batch = 65;
    CHECK(validate_config(&bad) == MOE_ERR_UNSUPPORTED);
    bad = named[0];
    bad.max_top_k = 897;
    CHECK(validate_config(&bad) == MOE_ERR_INVALID_ARG);
    bad = named[0];
    bad.hidden = 7100;
    CHECK(validate_config(&bad) == MOE_ERR_UNSUPPORTED);
    bad = named[0];
    bad.n_experts = 1056;
    CHECK(validate_config(&bad) == MOE_ERR_UNSUPPORTED);
    bad = named[0];
    bad.router_dtype = 7;
    CHECK(validate_config(&bad) == MOE_ERR_INVALID_ARG);
    CHECK(validate_config(nullptr) == MOE_ERR_INVALID_ARG);
    // A seeded sweep of random configurations.
    const std::vector<int> dims = {128, 256, 384, 512, 640, 1024, 1152, 2048, 3072, 4096,
                                   6144, 7168, 8192, 9216, 16384, 100, 0, -128};
    const std::vector<int> experts = {32, 64, 96, 256, 896, 1024, 1056, 48, 0};
    int valid = 0;
    for (int i = 0; i < 3000; ++i) {
        moe_decode_config c;
        c.hidden = pick(dims);
        c.latent = pick(dims);
        c.n_experts = pick(experts);
        c.expert_inter = pick(dims);
        c.shared_inter = pick(dims);
        c.max_batch = 1 + (int)(next_u32() % 70);
        c.max_top_k = 1 + (int)(next_u32() % 70);
        c.router_dtype = (int)(next_u32() % 3);
        const moe_status st = validate_config(&c);
        CHECK(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED);
        if (st != MOE_OK) continue;
        ++valid;
        CHECK(c.max_batch <= kMaxBatch && c.max_top_k <= kMaxTopK && c.max_top_k <= c.n_experts);
        check_layout(c);
        if (i % 10 == 0) check_plans(c);
    }
    CHECK(valid > 50);
    std::printf("plan_check: %d random configurations valid, %d failures\n", valid, failures);
    return failures ? 1 : 0;
}
