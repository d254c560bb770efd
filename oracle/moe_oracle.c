/*
 * moe_oracle.c - plain, slow, binary64 CPU oracle of the sparse latent-MoE
 * decode step (router scoring, top-k selection with renormalised weights,
 * latent down-projection, MXFP4 SwiGLU experts, weighted combine, bf16 shared
 * expert, latent up-projection).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never calls it, and the two share no source, header, table or helper.
 *
 * Sources of what is computed:
 *  - Kimi K3 layer shape (896 experts, 16 active per token, experts stored
 *    natively as MXFP4): page "快是可以生成的，可信只能证明（vLLM 重写 Kimi K3
 *    解码路径…）", section "为什么一条请求会慢"; page "NVIDIA uses a 12,000-line
 *    Megakernel to optimize Kimi K3 inference…", section "一个工程师、1.2万行代码、
 *    AI辅助开发".
 *  - Router scoring, latent projection and a shared expert as separate parts of
 *    the MoE layer: page "快是可以生成的，可信只能证明", section "他们换掉了什么"
 *    (third item of the list).
 *  - MXFP4 = OCP Microscaling (MX) v1.0: blocks of 32 E2M1 elements sharing one
 *    E8M0 power-of-two scale.
 *  - Everything the pages leave open (sigmoid scores, a per-expert bias that
 *    only moves the selection key, renormalisation over the chosen k, SwiGLU,
 *    nibble order, bf16 rounding points) is a stated reading of the layer
 *    definition; each reading is marked READING below.
 *
 * Conventions: every weight row is contiguous along its reduction dimension
 * (y = W x).  bf16 values are passed as their 16-bit patterns.  All sums are
 * plain left-to-right binary64 loops; no blocking, no reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t hidden;        /* H  */
    int32_t latent;        /* L  */
    int32_t n_experts;     /* E  */
    int32_t expert_inter;  /* I  */
    int32_t shared_inter;  /* Is */
    int32_t top_k;         /* k  */
    int32_t router_is_f32; /* 1: router weights are binary32, 0: bf16 */
} oracle_dims;

typedef struct {           /* every pointer optional (NULL = not wanted)   */
    double  *logit;        /* [B][E]       router logits                    */
    double  *score;        /* [B][E]       sigmoid scores                   */
    double  *key;          /* [B][E]       selection keys s + bias          */
    int32_t *idx;          /* [B][k]       chosen experts, ascending id     */
    double  *weight;       /* [B][k]       renormalised weights             */
    double  *z;            /* [B][L]       latent input of the experts      */
    double  *act;          /* [B][k][I]    SwiGLU activation per chosen slot */
    double  *ylat;         /* [B][L]       weighted combine in latent space */
    double  *ash;          /* [B][Is]      shared-expert SwiGLU activation   */
    double  *sh;           /* [B][H]       shared-expert output              */
    double  *up;           /* [B][H]       latent up-projection of ylat      */
    double  *out;          /* [B][H]       layer output                      */
} oracle_outputs;

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* FP4 E2M1 (OCP MX v1.0): sign, 2 exponent bits with bias 1, 1 mantissa bit.
 * Code 0x8 is negative zero. */
static const double kE2M1[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

double oracle_e2m1_value(int32_t code) { return kE2M1[code & 15]; }

/* E8M0 scale (OCP MX v1.0): the byte is a biased exponent, value 2^(byte-127);
 * 0xFF is NaN. */
double oracle_e8m0_value(int32_t byte)
{
    if ((byte & 255) == 255) return NAN;
    return ldexp(1.0, (byte & 255) - 127);
}

/* bf16 pattern -> value (exact). */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 value straight to the nearest bf16 (ties to even) and
 * return the bit pattern.  bf16 keeps 8 significant bits: for |v| in
 * [2^(e-1), 2^e) its spacing is 2^(e-8); below 2^-126 the spacing stays
 * 2^-133 (subnormals).  No intermediate rounding to binary32. */
uint16_t oracle_bf16_bits_rne(double v)
{
    if (isnan(v)) return 0x7FC0;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isinf(v)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m 2^e, m in [0.5, 1) */
    int q = e - 8;                      /* exponent of the bf16 spacing */
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(a, -q)), q); /* round-to-nearest-even */
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80); /* overflow -> inf */
    float f = (float)r;                 /* exact: r is representable in bf16 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

double oracle_bf16_round(double v) { return oracle_bf16_value(oracle_bf16_bits_rne(v)); }

/* Element j of an MXFP4 row: code in byte j/2, low nibble for even j
 * (READING: the pages say only "MXFP4"), scaled by byte j/32 of the row's
 * E8M0 scale array. */
double oracle_mxfp4_element(const uint8_t *q_row, const uint8_t *s_row, int32_t j)
{
    uint8_t byte = q_row[j / 2];
    int code = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return kE2M1[code] * oracle_e8m0_value(s_row[j / 32]);
}

static double sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }

/* ------------------------------------------------------------------------- */
/* Dot products: one output row at a time, left-to-right                      */
/* ------------------------------------------------------------------------- */

static double dot_bf16(const uint16_t *w, const double *v, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i) acc += oracle_bf16_value(w[i]) * v[i];
    return acc;
}

static double dot_f32(const float *w, const double *v, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i) acc += (double)w[i] * v[i];
    return acc;
}

static double dot_mxfp4(const uint8_t *q_row, const uint8_t *s_row, const double *v, int32_t n)
{
    double acc = 0.0;
    for (int32_t j = 0; j < n; ++j) acc += oracle_mxfp4_element(q_row, s_row, j) * v[j];
    return acc;
}

/* ------------------------------------------------------------------------- */
/* Routing                                                                    */
/* ------------------------------------------------------------------------- */

/* Router scores for B tokens: logit_e = Wr[e] . x, score_e = sigmoid(logit_e)
 * (READING: sigmoid scoring).  logit may be NULL. */
int32_t oracle_router_scores(const oracle_dims *d, int32_t B, const uint16_t *x,
                             const void *router_w, double *logit, double *score)
{
    const int64_t H = d->hidden, E = d->n_experts;
    double *xv = malloc(sizeof(double) * H);
    if (!xv) return -1;
    for (int32_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) xv[h] = oracle_bf16_value(x[b * H + h]);
        for (int64_t e = 0; e < E; ++e) {
            double l = d->router_is_f32
                           ? dot_f32((const float *)router_w + e * H, xv, H)
                           : dot_bf16((const uint16_t *)router_w + e * H, xv, H);
            if (logit) logit[b * E + e] = l;
            score[b * E + e] = sigmoid(l);
        }
    }
    free(xv);
    return 0;
}

typedef struct {
    double key;
    int32_t id;
} keyed_expert;

/* Total order used for selection: larger key first, equal keys -> lower id. */
static int by_key_desc_then_id(const void *pa, const void *pb)
{
    const keyed_expert *a = pa, *b = pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static int by_id(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Top-k of E keys: sort all E experts by (key descending, id ascending), keep
 * the first k, return them in ascending id. */
int32_t oracle_topk(const double *key, int32_t E, int32_t k, int32_t *idx_out)
{
    if (k < 1 || k > E) return -1;
    keyed_expert *order = malloc(sizeof(keyed_expert) * (size_t)E);
    if (!order) return -1;
    for (int32_t e = 0; e < E; ++e) {
        order[e].key = key[e];
        order[e].id = e;
    }
    qsort(order, (size_t)E, sizeof(keyed_expert), by_key_desc_then_id);
    for (int32_t j = 0; j < k; ++j) idx_out[j] = order[j].id;
    qsort(idx_out, (size_t)k, sizeof(int32_t), by_id);
    free(order);
    return 0;
}

/* Selection and weights for B tokens from their scores.
 *   key_e = score_e + bias_e   in binary64 (READING: the bias moves only the
 *                              selection key)
 *   S     = top-k by key (full sort; ties -> lower id), or forced_idx when
 *           given
 *   w_e   = score_e / sum_{j in S} score_j  (READING: unbiased scores,
 *                                            renormalised, no extra factor)
 * bias may be NULL (zero).  key / weight may be NULL. */
int32_t oracle_select(const oracle_dims *d, int32_t B, const double *score, const float *bias,
                      const int32_t *forced_idx, double *key, int32_t *idx, double *weight)
{
    const int32_t E = d->n_experts, k = d->top_k;
    double *kb = malloc(sizeof(double) * (size_t)E);
    if (!kb) return -1;
    for (int32_t b = 0; b < B; ++b) {
        const double *s = score + (int64_t)b * E;
        for (int32_t e = 0; e < E; ++e)
            kb[e] = s[e] + (bias ? (double)bias[e] : 0.0);
        if (key) memcpy(key + (int64_t)b * E, kb, sizeof(double) * (size_t)E);
        int32_t *sel = idx + (int64_t)b * k;
        if (forced_idx) {
            memcpy(sel, forced_idx + (int64_t)b * k, sizeof(int32_t) * (size_t)k);
            qsort(sel, (size_t)k, sizeof(int32_t), by_id);
        } else if (oracle_topk(kb, E, k, sel) != 0) {
            free(kb);
            return -1;
        }
        double total = 0.0;
        for (int32_t j = 0; j < k; ++j) total += s[sel[j]];
        if (weight)
            for (int32_t j = 0; j < k; ++j) weight[(int64_t)b * k + j] = s[sel[j]] / total;
    }
    free(kb);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The whole layer step                                                       */
/* ------------------------------------------------------------------------- */

/* Rounding policy (the layer definition fixes only "bf16 output, f32
 * accumulation"; where intermediates are rounded is an implementation choice):
 *   ORACLE_ROUND_NONE    = 0: every value stays binary64, output included;
 *   ORACLE_ROUND_OUTPUT  = 1: intermediates stay binary64, the output is
 *                             rounded to bf16 (the GPU library keeps its
 *                             intermediates at f32-grade precision);
 *   ORACLE_ROUND_BF16_ALL = 2: z, the expert activations, the combined latent,
 *                             the shared activation and the output are each
 *                             rounded to bf16 where they are produced.
 * Tokens are independent; each is processed on its own. */
enum { ORACLE_ROUND_NONE = 0, ORACLE_ROUND_OUTPUT = 1, ORACLE_ROUND_BF16_ALL = 2 };
int32_t oracle_moe_step(const oracle_dims *d, int32_t B, const uint16_t *x, const void *router_w,
                        const float *bias, const uint16_t *lat_down, const uint16_t *lat_up,
                        const uint8_t *w13_q, const uint8_t *w13_s, const uint8_t *w2_q,
                        const uint8_t *w2_s, const uint16_t *sh_w13, const uint16_t *sh_w2,
                        int32_t rounding, const int32_t *forced_idx, oracle_outputs *o)
{
    const int64_t H = d->hidden, L = d->latent, E = d->n_experts, I = d->expert_inter,
                  Is = d->shared_inter, k = d->top_k;
    if (H < 1 || L < 1 || E < 1 || I < 1 || Is < 1 || k < 1 || k > E || B < 1) return -1;
    if (L % 32 || I % 32) return -1; /* whole MX blocks per row */
    if (rounding < ORACLE_ROUND_NONE || rounding > ORACLE_ROUND_BF16_ALL) return -1;
    const int mid = rounding == ORACLE_ROUND_BF16_ALL; /* round intermediates */
    const int fin = rounding != ORACLE_ROUND_NONE;     /* round the output   */

    double *score = malloc(sizeof(double) * E);
    double *logit = malloc(sizeof(double) * E);
    int32_t *sel = malloc(sizeof(int32_t) * k);
    double *wsel = malloc(sizeof(double) * k);
    double *xv = malloc(sizeof(double) * H);
    double *z = malloc(sizeof(double) * L);
    double *a = malloc(sizeof(double) * I);
    double *ye = malloc(sizeof(double) * L);
    double *ylat = malloc(sizeof(double) * L);
    double *as = malloc(sizeof(double) * Is);
    double *sh = malloc(sizeof(double) * H);
    int32_t rc = 0;
    if (!score || !logit || !sel || !wsel || !xv || !z || !a || !ye || !ylat || !as || !sh) {
        rc = -1;
        goto done;
    }

    for (int32_t b = 0; b < B; ++b) {
        const uint16_t *xb = x + b * H;
        for (int64_t h = 0; h < H; ++h) xv[h] = oracle_bf16_value(xb[h]);

        /* Router: scores, selection, renormalised weights. */
        if (oracle_router_scores(d, 1, xb, router_w, logit, score) != 0 ||
            oracle_select(d, 1, score, bias, forced_idx ? forced_idx + b * k : NULL,
                          o->key ? o->key + b * E : NULL, sel, wsel) != 0) {
            rc = -1;
            goto done;
        }
        if (o->logit) memcpy(o->logit + b * E, logit, sizeof(double) * E);
        if (o->score) memcpy(o->score + b * E, score, sizeof(double) * E);
        if (o->idx) memcpy(o->idx + b * k, sel, sizeof(int32_t) * k);
        if (o->weight) memcpy(o->weight + b * k, wsel, sizeof(double) * k);

        /* Latent down-projection: z = W_ld x. */
        for (int64_t l = 0; l < L; ++l) {
            double v = dot_bf16(lat_down + l * H, xv, H);
            z[l] = mid ? oracle_bf16_round(v) : v;
        }
        if (o->z) memcpy(o->z + b * L, z, sizeof(double) * L);

        /* Chosen experts, in ascending id: SwiGLU in latent space, then the
         * weighted sum of their down-projections. */
        for (int64_t l = 0; l < L; ++l) ylat[l] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const int64_t e = sel[j];
            const uint8_t *q13 = w13_q + e * (2 * I) * (L / 2);
            const uint8_t *s13 = w13_s + e * (2 * I) * (L / 32);
            for (int64_t i = 0; i < I; ++i) {
                double g = dot_mxfp4(q13 + i * (L / 2), s13 + i * (L / 32), z, (int32_t)L);
                double u = dot_mxfp4(q13 + (I + i) * (L / 2), s13 + (I + i) * (L / 32), z,
                                     (int32_t)L);
                double v = g * sigmoid(g) * u; /* silu(gate) * up */
                a[i] = mid ? oracle_bf16_round(v) : v;
            }
            if (o->act) memcpy(o->act + (b * k + j) * I, a, sizeof(double) * I);
            const uint8_t *q2 = w2_q + e * L * (I / 2);
            const uint8_t *s2 = w2_s + e * L * (I / 32);
            for (int64_t l = 0; l < L; ++l)
                ye[l] = dot_mxfp4(q2 + l * (I / 2), s2 + l * (I / 32), a, (int32_t)I);
            for (int64_t l = 0; l < L; ++l) ylat[l] += wsel[j] * ye[l];
        }
        if (mid)
            for (int64_t l = 0; l < L; ++l) ylat[l] = oracle_bf16_round(ylat[l]);
        if (o->ylat) memcpy(o->ylat + b * L, ylat, sizeof(double) * L);

        /* Shared expert on the hidden state (READING: weight 1, no gate). */
        for (int64_t i = 0; i < Is; ++i) {
            double g = dot_bf16(sh_w13 + i * H, xv, H);
            double u = dot_bf16(sh_w13 + (Is + i) * H, xv, H);
            double v = g * sigmoid(g) * u;
            as[i] = mid ? oracle_bf16_round(v) : v;
        }
        if (o->ash) memcpy(o->ash + b * Is, as, sizeof(double) * Is);
        for (int64_t h = 0; h < H; ++h) sh[h] = dot_bf16(sh_w2 + h * Is, as, Is);
        if (o->sh) memcpy(o->sh + b * H, sh, sizeof(double) * H);

        /* Back to the hidden size, plus the shared expert. */
        for (int64_t h = 0; h < H; ++h) {
            double u = dot_bf16(lat_up + h * L, ylat, L);
            if (o->up) o->up[b * H + h] = u;
            double v = u + sh[h];
            if (o->out) o->out[b * H + h] = fin ? oracle_bf16_round(v) : v;
        }
    }

done:
    free(score);
    free(logit);
    free(sel);
    free(wsel);
    free(xv);
    free(z);
    free(a);
    free(ye);
    free(ylat);
    free(as);
    free(sh);
    return rc;
}
