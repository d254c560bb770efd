/*
 * oracle_check.c - runs the CPU oracle (moe_oracle.c, compiled into this
 * program) under the address and undefined-behaviour sanitizers: every entry
 * point on small seeded layers, every rounding policy, bf16 and f32 routers,
 * with and without a bias and a forced selection, k from 1 to E, and the
 * argument checks.  Exits non-zero on a failed check; the sanitizers abort on
 * an out-of-bounds access, a leak or undefined behaviour.
 */
#include "../../oracle/moe_oracle.c"

#include <stdio.h>

static int failures = 0;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);       \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

static uint64_t state = 88172645463325252ull;
static uint32_t next_u32(void) /* xorshift64* */
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}
static double uniform(void) { return (next_u32() + 0.5) / 4294967296.0; }
static uint16_t bf16_small(void) { return oracle_bf16_bits_rne((uniform() - 0.5) * 0.2); }

static void run_layer(int32_t H, int32_t L, int32_t E, int32_t I, int32_t Is, int32_t k,
                      int32_t f32_router, int32_t B)
{
    oracle_dims d = {H, L, E, I, Is, k, f32_router};
    uint16_t *x = malloc(sizeof(uint16_t) * B * H);
    void *rw = malloc((f32_router ? 4 : 2) * (size_t)E * H);
    float *bias = malloc(sizeof(float) * E);
    uint16_t *ld = malloc(sizeof(uint16_t) * L * H), *lu = malloc(sizeof(uint16_t) * H * L);
    uint8_t *q13 = malloc((size_t)E * 2 * I * L / 2), *s13 = malloc((size_t)E * 2 * I * L / 32);
    uint8_t *q2 = malloc((size_t)E * L * I / 2), *s2 = malloc((size_t)E * L * I / 32);
    uint16_t *sh13 = malloc(sizeof(uint16_t) * 2 * Is * H), *sh2 = malloc(sizeof(uint16_t) * H * Is);
    for (int64_t i = 0; i < (int64_t)B * H; ++i) x[i] = oracle_bf16_bits_rne(uniform() * 2 - 1);
    for (int64_t i = 0; i < (int64_t)E * H; ++i) {
        if (f32_router) ((float *)rw)[i] = (float)((uniform() - 0.5) * 0.2);
        else ((uint16_t *)rw)[i] = bf16_small();
    }
    for (int32_t e = 0; e < E; ++e) bias[e] = (float)((uniform() - 0.5) * 0.1);
    for (int64_t i = 0; i < (int64_t)L * H; ++i) { ld[i] = bf16_small(); lu[i] = bf16_small(); }
    for (int64_t i = 0; i < (int64_t)E * I * L; ++i) q13[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < (int64_t)E * 2 * I * L / 32; ++i) s13[i] = (uint8_t)(118 + next_u32() % 5);
    for (int64_t i = 0; i < (int64_t)E * L * I / 2; ++i) q2[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < (int64_t)E * L * I / 32; ++i) s2[i] = (uint8_t)(118 + next_u32() % 5);
    for (int64_t i = 0; i < (int64_t)2 * Is * H; ++i) sh13[i] = bf16_small();
    for (int64_t i = 0; i < (int64_t)H * Is; ++i) sh2[i] = bf16_small();

    double *logit = malloc(sizeof(double) * B * E), *score = malloc(sizeof(double) * B * E);
    double *key = malloc(sizeof(double) * B * E), *w = malloc(sizeof(double) * B * k);
    int32_t *idx = malloc(sizeof(int32_t) * B * k), *forced = malloc(sizeof(int32_t) * B * k);
    double *z = malloc(sizeof(double) * B * L), *act = malloc(sizeof(double) * B * k * I);
    double *ylat = malloc(sizeof(double) * B * L), *ash = malloc(sizeof(double) * B * Is);
    double *sh = malloc(sizeof(double) * B * H), *up = malloc(sizeof(double) * B * H);
    double *out = malloc(sizeof(double) * B * H);
    oracle_outputs all = {logit, score, key, idx, w, z, act, ylat, ash, sh, up, out};
    oracle_outputs only_out = {0};
    only_out.out = out;
    /* forced selections: k distinct experts per token */
    for (int32_t b = 0; b < B; ++b)
        for (int32_t j = 0; j < k; ++j) forced[b * k + j] = (int32_t)(((int64_t)j * (E / k) + b) % E);
    for (int32_t rounding = 0; rounding <= 2; ++rounding) {
        CHECK(oracle_moe_step(&d, B, x, rw, bias, ld, lu, q13, s13, q2, s2, sh13, sh2, rounding,
                              NULL, &all) == 0);
        for (int64_t i = 0; i < (int64_t)B * H; ++i) CHECK(isfinite(out[i]));
        for (int32_t b = 0; b < B; ++b) {
            double t = 0;
            for (int32_t j = 0; j < k; ++j) t += w[b * k + j];
            CHECK(fabs(t - 1.0) < 1e-12);
            for (int32_t j = 1; j < k; ++j) CHECK(idx[b * k + j] > idx[b * k + j - 1]);
        }
        CHECK(oracle_moe_step(&d, B, x, rw, NULL, ld, lu, q13, s13, q2, s2, sh13, sh2, rounding,
                              forced, &only_out) == 0);
    }
    CHECK(oracle_router_scores(&d, B, x, rw, NULL, score) == 0);
    CHECK(oracle_select(&d, B, score, bias, NULL, NULL, idx, NULL) == 0);
    CHECK(oracle_select(&d, B, score, NULL, forced, key, idx, w) == 0);
    int32_t *all_ids = malloc(sizeof(int32_t) * E);
    CHECK(oracle_topk(key, E, E, all_ids) == 0);
    for (int32_t e = 0; e < E; ++e) CHECK(all_ids[e] == e);
    free(all_ids);
    /* argument checks */
    oracle_dims bad = d;
    bad.top_k = E + 1;
    CHECK(oracle_moe_step(&bad, B, x, rw, bias, ld, lu, q13, s13, q2, s2, sh13, sh2, 1, NULL,
                          &all) == -1);
    bad = d;
    bad.latent = L + 16;
    CHECK(oracle_moe_step(&bad, B, x, rw, bias, ld, lu, q13, s13, q2, s2, sh13, sh2, 1, NULL,
                          &all) == -1);
    CHECK(oracle_moe_step(&d, B, x, rw, bias, ld, lu, q13, s13, q2, s2, sh13, sh2, 3, NULL,
                          &all) == -1);
    CHECK(oracle_topk(key, E, 0, idx) == -1 && oracle_topk(key, E, E + 1, idx) == -1);

    free(x); free(rw); free(bias); free(ld); free(lu); free(q13); free(s13); free(q2);
    free(s2); free(sh13); free(sh2); free(logit); free(score); free(key); free(w); free(idx);
    free(forced); free(z); free(act); free(ylat); free(ash); free(sh); free(up); free(out);
}

int main(void)
{
    /* format helpers over their whole domains */
    for (int c = 0; c < 16; ++c) CHECK(fabs(oracle_e2m1_value(c)) <= 6.0);
    for (int b = 0; b < 255; ++b) CHECK(oracle_e8m0_value(b) > 0.0);
    CHECK(isnan(oracle_e8m0_value(255)));
    for (uint32_t p = 0; p < 65536; ++p) {
        double v = oracle_bf16_value((uint16_t)p);
        if (!isnan(v)) CHECK(oracle_bf16_bits_rne(v) == (uint16_t)p || v == 0.0);
    }
    run_layer(64, 64, 8, 32, 64, 2, 0, 3);
    run_layer(128, 64, 32, 64, 128, 6, 1, 2);
    run_layer(64, 32, 8, 32, 32, 8, 0, 1);   /* k = E */
    run_layer(64, 32, 8, 32, 32, 1, 1, 4);   /* k = 1 */
    printf("oracle_check: %d failures\n", failures);
    return failures ? 1 : 0;
}
