/*
 * moe_decode.h - C ABI of the MI355X (gfx950) decode step of a sparse latent
 * mixture-of-experts layer.
 *
 * What one step computes, for each of B tokens x (bf16, hidden size H):
 *   1. router scores s_e = sigmoid(Wr[e] . x) over E experts; selection key
 *      s_e + bias_e; the k experts with the largest keys (equal keys: lower id
 *      first); weights w_e = s_e / sum of the k selected s;
 *   2. latent input z = W_ld x (H -> L);
 *   3. for each selected expert, MXFP4 SwiGLU in latent space:
 *      a = silu(W13_e[0:I] z) * (W13_e[I:2I] z), y_e = W2_e a;
 *   4. weighted combine in latent space ylat = sum_e w_e y_e;
 *   5. shared expert on x: ash = silu(S13[0:Is] x) * (S13[Is:2Is] x), sh = S2 ash;
 *   6. out = bf16_rne(W_lu ylat + sh)  (L -> H, plus the shared expert).
 *
 * Sources.  The layer shape (896 experts, 16 active per token, expert weights
 * stored natively as MXFP4) is stated on the page "快是可以生成的，可信只能证明
 * （vLLM 重写 Kimi K3 解码路径，以及怎么放心合并 Agent 写的内核）", section
 * "为什么一条请求会慢", and on the page "NVIDIA uses a 12,000-line Megakernel to
 * optimize Kimi K3 inference, and vLLM says AI code is now faster than human
 * review", section "一个工程师、1.2万行代码、AI辅助开发".  Router scoring, the
 * latent projection and the shared expert as parts of the MoE layer are named
 * on the first page, section "他们换掉了什么" (third item).  MXFP4 is the OCP
 * Microscaling v1.0 format: blocks of 32 E2M1 codes sharing one E8M0 scale.
 * Sigmoid scoring, the bias acting on the selection key only, renormalisation
 * without an extra factor, SwiGLU, the nibble order and the rounding policy are
 * readings of a layer definition the pages leave open.
 *
 * Layouts (row-major; every weight row is contiguous along its reduction
 * dimension, i.e. y = W x):
 *   x, out    bf16 [B][H]
 *   router_w  bf16 [E][H]  (or f32 [E][H], see router_dtype)
 *   bias      f32  [E], or NULL for zero bias
 *   lat_down  bf16 [L][H]          lat_up  bf16 [H][L]
 *   w13_q     u8 [E][2I][L/2]      two E2M1 codes per byte; element 2j in the
 *                                  low nibble, 2j+1 in the high nibble; rows
 *                                  0..I-1 gate, I..2I-1 up
 *   w13_s     u8 [E][2I][L/32]     E8M0 scale byte of each 32-element block
 *   w2_q      u8 [E][L][I/2]       w2_s u8 [E][L][I/32]
 *   sh_w13    bf16 [2Is][H]        gate rows then up rows
 *   sh_w2     bf16 [H][Is]
 *   topk_idx  i32 [B][k]  selected expert ids in ascending order
 *   topk_w    f32 [B][k]  their renormalised weights, aligned with topk_idx
 * bf16 values are passed as uint16_t bit patterns.
 *
 * Precision.  Products and sums are formed in f32 (bf16 x bf16 products are
 * exact in f32; MXFP4 elements are exact in bf16).  Intermediates (z, the
 * expert activations, ylat, the shared activation) are carried as a pair of
 * bf16 values hi + lo (about 16 significant bits) into the next contraction;
 * the output is rounded to bf16 once, to nearest even.  The top-k decision is
 * taken on f32 keys.
 *
 * Ownership.  Every pointer is borrowed.  Weights must stay alive and unchanged
 * until moe_decode_destroy.  The workspace (device memory of at least
 * moe_decode_workspace_size bytes, 256-byte aligned) belongs to the context
 * until destroy.  Several contexts, of the same or of different
 * configurations, may share one workspace (at least the largest of their
 * sizes) when their steps are ordered on one stream: the counters every step
 * returns to zero sit at the same offsets for every configuration, and the
 * rest of the workspace only carries values within one step.  Contexts that
 * share a workspace also share its fault flag (moe_decode_read_flags).  The
 * library never allocates device memory.
 *
 * Errors.  Every call returns a moe_status; nothing is thrown, printed or
 * aborted.  After MOE_ERR_HIP the HIP error code is kept in the context
 * (moe_decode_last_hip_error).
 *
 * Asynchrony.  moe_decode_step only enqueues work on the given stream: no host
 * synchronisation, no allocation, no memset; it may be captured into a HIP
 * graph.  A context is not thread-safe.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *moe_stream_t; /* == hipStream_t; NULL = default stream */

typedef struct moe_decode_ctx moe_decode_ctx;     /* opaque, library-owned host object */
typedef struct moe_decode_graph moe_decode_graph; /* opaque captured multi-layer step */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, batch/top_k out of range, misalignment */
    MOE_ERR_UNSUPPORTED = -2, /* shape the kernels do not cover, or device is not gfx950 */
    MOE_ERR_HIP = -3,         /* a HIP runtime call failed (see last_hip_error) */
    MOE_ERR_WORKSPACE = -4    /* workspace missing, too small or misaligned */
} moe_status;

enum { MOE_ROUTER_BF16 = 0, MOE_ROUTER_F32 = 1 };

/* Layer dimensions, all in elements.  Supported: H, L, I, Is multiples of 128
 * such that each of H, L, I and L + Is is 128 * KW * S with KW in {1, 2, 4, 8}
 * and S <= 8 (at most 8192 elements); E a multiple of 32 and at most 1024;
 * 1 <= max_batch <= 64; 1 <= max_top_k <= min(E, 64). */
typedef struct {
    int32_t hidden;       /* H  */
    int32_t latent;       /* L  */
    int32_t n_experts;    /* E  */
    int32_t expert_inter; /* I  */
    int32_t shared_inter; /* Is */
    int32_t max_batch;    /* largest B a step may use */
    int32_t max_top_k;    /* largest k a step may use */
    int32_t router_dtype; /* MOE_ROUTER_BF16 or MOE_ROUTER_F32 */
} moe_decode_config;

/* Device pointers, borrowed; every pointer 16-byte aligned.  Scale bytes must
 * lie in 1..254 (0x00 and the NaN code 0xFF are outside the contract). */
typedef struct {
    const void *router_w;    /* [E][H] bf16 or f32 */
    const float *router_bias;/* [E] f32, or NULL */
    const uint16_t *lat_down;/* [L][H] bf16 */
    const uint16_t *lat_up;  /* [H][L] bf16 */
    const uint8_t *w13_q;    /* [E][2I][L/2] */
    const uint8_t *w13_s;    /* [E][2I][L/32] */
    const uint8_t *w2_q;     /* [E][L][I/2] */
    const uint8_t *w2_s;     /* [E][L][I/32] */
    const uint16_t *sh_w13;  /* [2Is][H] bf16 */
    const uint16_t *sh_w2;   /* [H][Is] bf16 */
} moe_decode_weights;

/* Host only: checks a configuration against the supported shapes. */
moe_status moe_decode_validate_config(const moe_decode_config *cfg);

/* Host only: workspace bytes a context of this configuration needs (0 when
 * the configuration is invalid). */
size_t moe_decode_workspace_size(const moe_decode_config *cfg);

/* Creates a context on the current HIP device.  Checks the configuration, the
 * weight pointers and the device (must be gfx950), carves the workspace and
 * clears its counters (one small kernel on the default stream, then waits for
 * it; so no step of another context may be in flight on a shared workspace).
 * On success *out receives the context. */
moe_status moe_decode_init(const moe_decode_config *cfg, const moe_decode_weights *weights,
                           void *workspace, size_t workspace_bytes, moe_decode_ctx **out);

/* One decode step for `batch` tokens with `top_k` experts per token:
 * x [batch][H] bf16 -> out [batch][H] bf16; topk_idx [batch][top_k] and
 * topk_w [batch][top_k] receive the routing when not NULL.  Requires
 * 1 <= batch <= max_batch and 1 <= top_k <= max_top_k.  Asynchronous on
 * `stream`; x must not change and out must not be read until the stream
 * reaches the end of the step. */
moe_status moe_decode_step(moe_decode_ctx *ctx, const uint16_t *x, int32_t batch, int32_t top_k,
                           uint16_t *out, int32_t *topk_idx, float *topk_w, moe_stream_t stream);

/* Releases the context (no device memory is freed: the library owns none). */
moe_status moe_decode_destroy(moe_decode_ctx *ctx);

const char *moe_decode_status_string(moe_status s);
int32_t moe_decode_last_hip_error(const moe_decode_ctx *ctx);

/* ---- HIP graph of a stack of layers ------------------------------------ */

/* Captures n_layers consecutive steps (layer i: ctxs[i], x[i] -> out[i]) into
 * one instantiated HIP graph.  The pointers are baked into the graph: replays
 * read x[i] and write out[i] (and idx[i], w[i] when the arrays are not NULL
 * and their entries are not NULL).  Capture uses a private stream; nothing
 * runs until moe_decode_graph_launch. */
moe_status moe_decode_graph_create(moe_decode_ctx *const *ctxs, int32_t n_layers,
                                   const uint16_t *const *x, int32_t batch, int32_t top_k,
                                   uint16_t *const *out, int32_t *const *topk_idx,
                                   float *const *topk_w, moe_decode_graph **graph);
moe_status moe_decode_graph_launch(moe_decode_graph *graph, moe_stream_t stream);
moe_status moe_decode_graph_destroy(moe_decode_graph *graph);

/* ---- A step that allocates nothing ------------------------------------ */

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid allocation.  The
 * four-launch step of moe_decode_step (same arguments, same results) for the
 * configuration *cfg and the weights *w, without a context and without a
 * caller workspace: the workspace is a static device array of
 * MOE_DECODE_STATIC_WORKSPACE_BYTES that the library holds on each device it
 * runs on until the process ends.  The call clears the array's counters with
 * a small kernel on `stream`, then enqueues the step there; it calls no
 * allocation routine and performs no host synchronisation (the first call on
 * a device also reads the device's properties and the array's address).
 * Returns MOE_ERR_WORKSPACE when the configuration needs a larger workspace
 * than the array (moe_decode_workspace_size: the K3-scale layer fits at
 * max_batch up to 64), and otherwise the errors of moe_decode_init and
 * moe_decode_step.  Every call on one device uses the same array, which keeps
 * the last call's contents: calls whose work may overlap on one device (other
 * streams, other threads) race and give wrong results; order them on one
 * stream. */
#define MOE_DECODE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
moe_status moe_decode_step_static(const moe_decode_config *cfg, const moe_decode_weights *weights,
                                  const uint16_t *x, int32_t batch, int32_t top_k, uint16_t *out,
                                  int32_t *topk_idx, float *topk_w, moe_stream_t stream);

/* ---- Introspection (tests and profiling) ------------------------------- */

/* Which kernel shapes the last step of a context used (the batch-dependent
 * choices), for tests that check a batch reaches the intended code path. */
typedef struct {
    int32_t batch, top_k;
    int32_t col_tiles;     /* 16-token column groups of the router / latent-down kernel */
    int32_t split_in;      /* waves of a workgroup splitting K: router / latent-down / shared gate-up */
    int32_t split_out;     /* ... latent-up + shared-down */
    int32_t split_w13;     /* ... expert gate/up */
    int32_t split_w2;      /* ... expert down (waves per tile) */
    int32_t grid_in, grid_w13, grid_w2, grid_out; /* workgroups launched */
    int32_t router_f32;    /* 1 when the f32 router kernel ran */
    int32_t n_kernels;     /* kernels launched by the step */
    int32_t fused;         /* 1: one persistent launch; 2: dense-in + persistent launch;
                              3: side stream; 0: four launches */
    int32_t grid_step;     /* workgroups of the persistent launch (0 for four launches) */
    int32_t out_staged;    /* four launches: 1 when the output launch staged its whole
                              column operand in LDS (at most two tokens), 2 when it
                              staged the latent part (at most eight tokens), else 0 */
    int32_t routing;       /* where the routing ran: 0 in the dense-in launch (the
                              workgroup that completed the router), 1 in routing units
                              of the dense-in launch (above 8 tokens), 2 at the start
                              of the gate/up launch, 3 in the f32 router kernel */
    int32_t ordered;       /* 1 when the latent combine ran in a fixed order
                              (MOE_MODE_ORDERED): the step's outputs are the same bits
                              from run to run */
    int32_t in_staged;     /* how the dense-in launch read x: 0 through the caches per
                              tile, 1 staged in LDS once per workgroup (at most two
                              tokens), 2 staged in LDS per row group and step with K
                              split into slices (above 16 tokens, and from 9 when
                              the launch fits one round of resident workgroups), 3
                              staged in LDS once per workgroup, 3 to 8 tokens when
                              the launch fits one workgroup per compute unit */
} moe_decode_dispatch_info;
moe_status moe_decode_last_dispatch(const moe_decode_ctx *ctx, moe_decode_dispatch_info *info);

/* Execution mode of a context's later steps.
 *   MOE_MODE_FOUR_LAUNCHES (the default): dense-in, expert gate/up, expert
 *     down, output.  The routing (top-k and unit records) runs at the end of
 *     the dense-in launch, or, for up to 8 tokens and 128 token-expert pairs
 *     when the dense-in launch fits in one round of resident workgroups, at
 *     the start of the gate/up launch (see MOE_MODE_LATE_ROUTING): in one
 *     round, a routing at the end would leave the memory idle;
 *   MOE_MODE_TWO_LAUNCHES: the dense-in launch, then one persistent launch
 *     whose workgroups take the expert gate/up, shared-down, expert down and
 *     latent-up units from a queue in dependency order and wait on completion
 *     counters instead of kernel boundaries;
 *   MOE_MODE_SIDE_STREAM: the shared expert on a second stream of the
 *     context, as [P-vLLM] "他们换掉了什么" places it: on the caller's stream
 *     dense-in for the router and latent-down rows (and the routing), expert
 *     gate/up, expert down; on the side stream the shared gate/up and
 *     shared-down launches, which depend on x alone; then, on the caller's
 *     stream after an event join, latent-up plus the shared sums.  The
 *     step stays capturable (fork and join are event record/wait pairs);
 *   MOE_MODE_FUSED: the whole step as one persistent launch of that kind
 *     (router, latent and shared units too), the single-launch design of
 *     [P-NV] "一个工程师、1.2万行代码、AI辅助开发";
 *   MOE_MODE_LATE_ROUTING: the four launches, with the routing of up to 8
 *     tokens (and at most 128 token-expert pairs) always at the start of the
 *     gate/up launch instead of at the end of the dense-in launch: the
 *     dense-in launch then only streams weights, and every gate/up workgroup
 *     selects the experts itself from the scores and keys in memory, once,
 *     then runs its units (other batches, and steps with a next-layer
 *     prefetch, route in the dense-in launch);
 *   MOE_MODE_DENSE_ROUTING: the four launches with the routing always in the
 *     dense-in launch;
 *   MOE_MODE_ORDERED: the four launches (routing placed as by default) with
 *     the latent combine in a fixed order: each pair's weighted down output
 *     goes to the workspace, and the last of a token's k contributions to a
 *     group of latent rows adds them in the order of the token's expert ids.
 *     Every reduction of the step then has a fixed order, so a step's outputs
 *     are the same bits from run to run (the other forms add the expert
 *     outputs with f32 atomics, whose order varies).  The price: a store,
 *     an arrival and, for the last arrival, a read of the k rows at the end
 *     of each down unit (about 1.3 us at batch 1, 2-8 % of the step at
 *     batch 8-64).
 * Shapes without a built persistent kernel (the f32 router, other expert
 * chunk shapes) run the four launches.  All modes compute the same values.
 * Returns MOE_ERR_INVALID_ARG for another mode.  Host-only. */
enum {
    MOE_MODE_FUSED = 0,
    MOE_MODE_FOUR_LAUNCHES = 1,
    MOE_MODE_TWO_LAUNCHES = 2,
    MOE_MODE_SIDE_STREAM = 3,
    MOE_MODE_LATE_ROUTING = 4,
    MOE_MODE_DENSE_ROUTING = 5,
    MOE_MODE_ORDERED = 6
};
moe_status moe_decode_set_mode(moe_decode_ctx *ctx, int32_t mode);

/* Next-layer prefetch, the one-GPU analogue of the side-stream weight
 * prefetch of [P-vLLM] "他们换掉了什么": while a step of ctx routes (the
 * memory then streams little), its dense-in launch reads next's router and
 * latent-down rows, so that they sit in the last-level cache when next's step
 * streams them.  The values are dropped; nothing is written.  next must stay
 * alive while ctx uses it (next = NULL switches the prefetch off; next ==
 * ctx is refused with MOE_ERR_INVALID_ARG).  Applies to the dense-in launch
 * of the four-launch and two-launch forms and to the routed side of the
 * side-stream form.  Host-only. */
moe_status moe_decode_set_next_layer(moe_decode_ctx *ctx, const moe_decode_ctx *next);

/* Reads the context's sticky fault flags into *flags (synchronous copy from
 * the workspace; call after the steps completed).  Bit 0 is set when a bounded
 * wait of any step on this workspace ran out: a persistent step's wait on a
 * completion counter, or, in the multi-launch forms, the wait of a routing
 * unit (batches above 8) or a prefetch unit for the router to complete, or of
 * an output sum unit (batches above 8) for its row group's K slices.  The
 * step then finished instead of hanging, and its outputs are invalid.  The
 * flag stays set for the life of the workspace.  A wait runs out
 * only when the GPU does not run the step's workgroups concurrently (e.g.
 * preemption), after about 50 ms.  0 means no fault. */
moe_status moe_decode_read_flags(moe_decode_ctx *ctx, uint32_t *flags);

/* Per-kernel timing.  With events set (n = 2 x the step's kernel count, see
 * moe_decode_dispatch_info.n_kernels; HIP event handles owned by the caller),
 * every later eager step launches kernel i with events[2i] and events[2i+1]
 * attached to its dispatch (hipExtLaunchKernel), so that their elapsed time is
 * the kernel's own execution time, as a kernel trace reports it.  n = 0
 * (events may be NULL) switches timing off.  Returns MOE_ERR_INVALID_ARG when
 * n fits none of the step's forms (8, or 10 with the f32 router, for four
 * launches; 12 or 14 with the side stream, in launch order: dense-in main,
 * shared gate/up, gate/up, down, shared-down, latent-up; 4 for two launches;
 * 2 for one); a step whose kernel count differs from n is not timed. */
moe_status moe_decode_set_timing_events(moe_decode_ctx *ctx, void *const *events, int32_t n);

/* Copies the intermediates of the last step out of the workspace as f32
 * (device pointers, each optional):
 *   score, key [B][E]; z [B][L]; act [B][k][I] (per token and selection slot);
 *   ylat [B][L]; ash [B][Is]; n_active [1] (distinct experts of the step).
 * Valid only after a step with this batch and top_k on the same stream and
 * before any other step that shares the workspace. */
typedef struct {
    float *score, *key, *z, *act, *ylat, *ash;
    int32_t *n_active;
} moe_decode_debug;
moe_status moe_decode_debug_export(moe_decode_ctx *ctx, int32_t batch, int32_t top_k,
                                   const moe_decode_debug *dbg, moe_stream_t stream);

/* Decodes n MXFP4 elements (codes q, scales s, n a multiple of 32) to f32 with
 * the same device routine the expert kernels use; for format tests. */
moe_status moe_decode_debug_dequant(const uint8_t *q, const uint8_t *s, int64_t n, float *out,
                                    moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
