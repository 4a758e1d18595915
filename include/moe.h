/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN layer.
 *
 * The layer, forward pass on a prompt of T tokens:
 *   1. route     each token keeps its k largest router logits; their weights
 *                are the softmax renormalised over those k (mini-AGI PR #3,
 *                minagi/pool.py, `requested(scores)`);
 *   2. capacity  an expert keeps at most `limit` pairs, first come by token
 *                index; the rest drop and add nothing (mini-AGI PR #3/#4,
 *                configs/strix_halo_large.yaml `capacity_factor`, and the
 *                `keep` filter in minagi/pool.py);
 *   3. dispatch  kept token-expert pairs grouped by expert (the argsort and
 *                bincount over expert ids in minagi/pool.py);
 *   4. experts   per expert: gathered rows times W_gate and W_up, clamped
 *                SwiGLU, times W_down (minagi/pool.py `experts()`; the clamp
 *                and the dequantise-once FP16 route for experts holding many
 *                rows from Strata PR #4366, "Problem and result" and
 *                "Approach"; a K-parallel tile for experts holding few pairs
 *                from TensorFold PR #1607, "What this changes");
 *   5. combine   y[t] = sum of the token's kept pairs' weighted outputs.
 *
 * Conventions for every call:
 *   - The caller owns all device memory: logits, x, weights, y and both
 *     workspaces (sizes from the *_workspace_bytes queries). The library only
 *     allocates a small host-side plan handle. Workspaces are caller-provided
 *     because buffer sizes that change every call fragmented the allocator on
 *     the mini-AGI PR #4 README's `expandable_segments` row.
 *   - Every device call is asynchronous on `stream` (a hipStream_t; NULL =
 *     the default stream). Nothing synchronises the host except
 *     moe_plan_stats_get and moe_phase_times.
 *   - Arguments are validated on the host before any launch. On a non-OK
 *     status nothing was launched (so y is untouched) unless the status is
 *     MOE_EHIP from a launch; moe_last_error() then names the cause.
 *   - Device pointers must be 16-byte aligned. Matrices are row-major and
 *     K-contiguous: W_gate, W_up are [E + n_shared, F, D], W_down is
 *     [E + n_shared, D, F], as the pages use them through W.transpose(1, 2).
 *   - Supported dtype pairs (x, W): (F32, F32), (BF16, BF16), (F16, F16),
 *     (F16, Q4B32), (F16, Q4A32), (F16, Q4A64). Anything else is
 *     MOE_EUNSUPPORTED, never a fallback.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument (sizes, pointers, alignment)    */
    MOE_EUNSUPPORTED = -2,  /* dtype combination or size the library lacks */
    MOE_EWORKSPACE = -3,    /* workspace smaller than the size query       */
    MOE_EHIP = -4           /* the HIP runtime reported an error           */
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_F16 = 2,
    /* 4-bit block weights: `data` is uint8 [.., N, K/2] holding two's-
     * complement nibbles (low nibble = even K index), `scales` is fp16
     * [.., N, K/32], one scale per 32 consecutive K values of a row; the
     * value is q * s. Weights only; x must be F16. */
    MOE_Q4B32 = 3,
    /* Affine 4-bit groups (the MLX 4-bit checkpoints of TensorFold PR
     * #1607, "group 32" / "group 64" in its tuner tables): `data` is uint8
     * [.., N, K/2] holding unsigned nibbles 0..15 (low nibble = even K
     * index), `scales` is fp16 [.., N, K/G, 2]: per group of G = 32 / 64
     * consecutive K values of a row, its scale s then its bias b; the value
     * is q * s + b. Weights only; x must be F16. */
    MOE_Q4A32 = 4,
    MOE_Q4A64 = 5
} moe_dtype;

/* Plan shape. 1 <= k <= E <= 1024; T >= 0; T*(k+1) < 2^31; n_shared in
 * {0, 1}: a shared expert (index E in the weights) sees every token with
 * weight 1 and never drops (TensorFold PR #1607 plans of 256 experts plus a
 * shared slot). capacity_factor >= 0 and finite; 0 means uncapped (the
 * pages' default), otherwise limit = max(1, floor(cf * T * k / E)). */
typedef struct {
    int32_t T, E, k, n_shared;
    float capacity_factor;
} moe_plan_desc;

/* Forward options; moe_options_default() fills the defaults.
 *   swiglu_limit      c of h = silu(min(g, c)) * clamp(u, -c, c); <= 0 turns
 *                     the clamp off. Default 7.0.
 *   splitk_max_pairs  S: bf16/f16 experts holding n <= S pairs run the
 *                     split-K (weight-streaming) tile, the rest the full
 *                     MFMA tile. An f32
 *                     bound compared exactly in f64 (TensorFold PR #1607,
 *                     "Why 3.5, and why a fraction"); 0 sends every expert
 *                     to the full tile, a huge value every expert to
 *                     split-K. Default 16, the switch point measured on
 *                     MI355X. Unless MOE_OPT_EXACT_ROUTES is set, a plan
 *                     whose full-tile experts would not fill one round of
 *                     the GPU's compute units (their 256-row tiles times
 *                     F / 128 column blocks < compute units) sends those of
 *                     them holding <= 256 pairs to split-K as well: the
 *                     full tile would leave most units idle.
 *   fat_rows          4-bit weights only: experts holding >= fat_rows pairs
 *                     are dequantised once to fp16 and run the full tile;
 *                     the rest run the fused-dequant split-K tile. <= 0 turns
 *                     the fat route off; 1..16 is raised to 17, the light
 *                     tiles owning experts of 16 rows or fewer (Strata PR
 *                     #4366, maintainer's review). Default 64.
 *   flags             MOE_OPT_PHASE_EVENTS records HIP events around each
 *                     forward phase on the stream it runs on (see
 *                     moe_phase_times); with any of the bits
 *                     MOE_OPT_PHASE_ONLY(p) also set, only those phases
 *                     (each pair of events makes the GPU drain the work
 *                     before it: a few microseconds a phase).
 *                     The SwiGLU output H of a bf16 layer is one bf16 value
 *                     (the pages' compute-dtype buffer) when the plan is
 *                     uncapped, and a bf16 pair hi + lo (hi = bf16(h),
 *                     lo = bf16(h - hi), about 16 significant bits, the down
 *                     projection multiplying both) when it is capped: a
 *                     capped plan's dropped pairs can leave most rows of y
 *                     at zero, which shrinks RMS(y) against the rounding
 *                     error of the others, and the pair keeps such a layer
 *                     within 2e-2 x RMS(ref). MOE_OPT_BF16_SPLIT_H forces
 *                     the pair, MOE_OPT_BF16_PLAIN_H the one value (with
 *                     both set, the pair).
 *                     MOE_OPT_EXACT_ROUTES applies the S rule alone.
 *                     By default a prompt with experts on both sides and
 *                     T k D F above 2^33 runs its thin-group launches on a
 *                     second stream of the same device, owned by the
 *                     library (default priority), forked from `stream`
 *                     after the route classification and joined back
 *                     before the combine, so they overlap the fat experts'
 *                     dequantisation and full tiles; the call still orders
 *                     after earlier work on `stream` and before later work
 *                     on it; the first such call on a device creates the
 *                     stream and two events (under graph capture, make it
 *                     before capturing). MOE_OPT_ONE_STREAM keeps every
 *                     launch on `stream`.
 *                     A one-token call (T = 1) on a bf16 / fp16 layer, or
 *                     on a 4-bit layer with fp16 x (weights decoded in
 *                     registers as the thin tiles decode them), runs two
 *                     matrix-vector launches instead of the split-K
 *                     tile and the combine: one token's experts are
 *                     distinct, each holds one pair (mini-AGI PR #3,
 *                     minagi/pool.py, the one-row case), so the call is
 *                     the chosen experts' weight stream, spread over every
 *                     compute unit; the second launch also sums the pairs
 *                     into y in the combine's order and precision (phases
 *                     3 and 5 of moe_phase_times; 6 is not used).
 *                     MOE_OPT_TILED_DECODE keeps such calls on the tile. */
typedef struct {
    float swiglu_limit;
    float splitk_max_pairs;
    int32_t fat_rows;
    int32_t flags;
} moe_options;

#define MOE_OPT_PHASE_EVENTS 1
#define MOE_OPT_BF16_PLAIN_H 2
#define MOE_OPT_EXACT_ROUTES 4
#define MOE_OPT_BF16_SPLIT_H 8
#define MOE_OPT_ONE_STREAM 16
#define MOE_OPT_TILED_DECODE 32
#define MOE_OPT_PHASE_SHIFT 16
#define MOE_OPT_PHASE_ONLY(p) ((int32_t)(1u << (MOE_OPT_PHASE_SHIFT + (p))))

/* One weight tensor. `scales` is NULL unless dtype is a 4-bit format; then
 * it is 4-byte aligned (MOE_Q4B32) or 8-byte aligned (the affine formats):
 * a lane reads two adjacent block parameters at once. */
typedef struct {
    int32_t dtype;
    const void *data;
    const void *scales;
} moe_weight;

typedef struct moe_plan moe_plan;   /* opaque host handle */

typedef struct {
    int64_t T, E, k, n_shared;
    int64_t limit;          /* -1 when uncapped                            */
    int64_t pairs;          /* T*k routed pairs before the drop            */
    int64_t kept;           /* routed pairs kept                           */
    int64_t dropped;        /* pairs - kept                                */
    int64_t touched;        /* routed experts holding >= 1 kept pair       */
    int64_t max_rows;       /* most kept pairs one routed expert holds     */
    int64_t nonfinite;      /* NaN logits seen (ordered below -inf)        */
    int64_t thin, full, fat;/* routed experts per forward route by the S
                               and fat_rows rules of the options passed to
                               moe_plan_stats_get (without the move of an
                               underfilled full route to split-K)         */
    double drop_fraction;   /* dropped / pairs (mini-AGI PR #3,
                               tools/bench_hw.py `dropped_share`)          */
} moe_plan_stats;

/* Device arrays of a plan, inside its workspace, for inspection. All int32
 * unless noted; P = offsets[E + n_shared]. */
typedef struct {
    const int32_t *topk_id;    /* [T, k] expert ids in rank order           */
    const float *topk_w;       /* [T, k] f32 weights, renormalised          */
    const int32_t *slot;       /* [T, k] earlier tokens choosing that expert*/
    const int32_t *tok2pair;   /* [T, k] position in the pair list, or -1   */
    const int32_t *counts;     /* [E + n_shared] kept pairs per expert      */
    const int32_t *offsets;    /* [E + n_shared + 1] exclusive scan         */
    const int32_t *pair_token; /* [P] token of each expert-sorted pair      */
    const float *pair_w;       /* [P] its weight (1 for the shared expert)  */
    const int64_t *stats;      /* [8] dropped, kept, nonfinite, touched,
                                  max_rows, 0, 0, 0                         */
} moe_plan_views;

/* --- plan: route + capacity + dispatch -------------------------------- */

/* Bytes of device workspace moe_plan_create needs; 0 on invalid desc. */
size_t moe_plan_workspace_bytes(const moe_plan_desc *desc);

/* Route `logits` (f32 [T, E], device) and build the dispatch plan into `ws`
 * (device, >= moe_plan_workspace_bytes, 256-byte aligned). Launches only;
 * no host sync. The plan handle refers into `ws`: keep both alive while the
 * plan is used, free the handle with moe_plan_destroy. Ties in the logits go
 * to the lower expert index; +0 and -0 are equal; NaN ranks below -inf. */
moe_status moe_plan_create(const moe_plan_desc *desc, const float *logits,
                           void *ws, size_t ws_bytes, void *stream,
                           moe_plan **out);

/* Copies the plan's counters to the host (synchronises `stream`). */
moe_status moe_plan_stats_get(const moe_plan *plan, const moe_options *opt,
                              moe_plan_stats *out, void *stream);

moe_status moe_plan_get_views(const moe_plan *plan, moe_plan_views *out);

void moe_plan_destroy(moe_plan *plan);

/* --- router: logits + statistics + plan in one call ------------------- */

/* Routing statistics of one call, device-resident, written asynchronously
 * (mini-AGI PR #3, minagi/pool.py, `requested(scores)`; p = softmax of a
 * token's logits over all E experts):
 *   kept_mass  mean over tokens of the p mass on the k chosen experts,
 *              before their weights are renormalised;
 *   want_k     mean over tokens of the fewest experts whose p, largest
 *              first, add up to at least 0.9 (counted per token, then
 *              averaged);
 *   z_loss     mean over tokens of logsumexp(logits[t])^2;
 *   balance    E * sum_e frac_e * mean_t p[t, e], frac_e the share of tokens
 *              whose first choice (rank 0) is e;
 *   aux        balance + z_weight * z_loss.
 * Means over T tokens; all zero when T == 0. */
typedef struct {
    float kept_mass, want_k, z_loss, balance, aux;
    float reserved[3];
} moe_route_stats;

/* Bytes of device workspace moe_route needs (the plan's, then scratch for
 * the statistics); 0 on invalid desc. */
size_t moe_route_workspace_bytes(const moe_plan_desc *desc, int32_t D);

/* The router and the plan in one call: logits[T, E] = x[T, D] . w_router[E,
 * D]^T (x and w_router of one dtype, MOE_F32 / MOE_BF16 / MOE_F16; fp32
 * accumulation) written to the caller's `logits` (f32, device), then the
 * plan of moe_plan_create over those logits into `ws` (the handle refers into
 * it as for moe_plan_create), then, if `stats` (device) or `token_want`
 * (device int32 [T]) is non-NULL, the routing statistics of those logits and
 * of the plan's choices. z_weight weighs the z-loss in `aux` (the pages'
 * default is 1e-3); it must be finite. D must be a multiple of 8 in
 * 8 .. 2^20; pointers
 * 16-byte aligned, ws 256-byte aligned. Launches only; no host sync.
 * Argument errors are found before any launch and leave every output
 * untouched. The statistics are the same bits from run to run (fixed-order
 * sums, no float atomics). flags: MOE_OPT_PHASE_EVENTS records HIP events
 * around the router kernel, the plan and the statistics (phases 7, 8, 9 of
 * moe_phase_times; MOE_OPT_PHASE_ONLY bits select among them); other bits
 * are ignored. */
moe_status moe_route(const moe_plan_desc *desc, const void *x, int32_t x_dtype,
                     const void *w_router, int32_t D, float z_weight,
                     float *logits, moe_route_stats *stats,
                     int32_t *token_want, void *ws, size_t ws_bytes,
                     int32_t flags, void *stream, moe_plan **out);

/* --- forward: experts + combine --------------------------------------- */

void moe_options_default(moe_options *opt);

/* Bytes of device workspace moe_forward needs for this plan, sizes, dtypes
 * and options (the dequantised fp16 copies of 4-bit fat experts included,
 * sized for the most fat experts the plan could hold); 0 if unsupported. */
size_t moe_forward_workspace_bytes(const moe_plan *plan, int32_t D, int32_t F,
                                   int32_t x_dtype, int32_t w_dtype,
                                   const moe_options *opt);

/* y[T, D] = the layer on x[T, D]. D and F must be multiples of 128. `opt`
 * may be NULL for the defaults. The plan must come from logits over the same
 * T tokens. y_dtype is MOE_F32 (the residual stream's precision: the pages
 * compute the dispatch buffer in the compute dtype and return the layer
 * output in the residual's fp32, mini-AGI PR #4, minagi/pool.py, the
 * compute-dtype comment) or x's dtype (one rounding of that f32 result).
 * Each kept pair's unweighted output is held in fp16 in an fp16 layer (the
 * precision of its fp16 SwiGLU input) and in f32 otherwise; the combine
 * multiplies it by the routing weight in f32 and sums in slot order. */
moe_status moe_forward(const moe_plan *plan, const void *x, int32_t x_dtype,
                       moe_weight w_gate, moe_weight w_up, moe_weight w_down,
                       int32_t D, int32_t F, void *y, int32_t y_dtype,
                       void *ws, size_t ws_bytes, const moe_options *opt,
                       void *stream);

/* Device buffers of moe_forward inside its workspace `ws`, for inspection
 * after a call with the same plan, sizes, dtypes and options (tests and
 * debugging); the pointers stay valid while `ws` does. P is the most pairs
 * the plan can hold, T * k + n_shared * T; a pair's row is its index in the
 * plan's expert-sorted pair list (offsets[e] + its slot).
 *   h, h_lo      [P, h_ld] SwiGLU output of the pairs of experts on the
 *                split-K (thin) routes, x's dtype; h_lo is the bf16 low
 *                plane (NULL unless the layer carries one);
 *   ht, ht_lo    [F / 32][P][32] SwiGLU output of the pairs of experts on the
 *                full tile (NULL when the layout has no full route);
 *   ypair        [P, D] each kept pair's unweighted expert output, fp16
 *                (ypair_dtype MOE_F16) in an fp16 layer, else f32;
 *   fat_slot     [E + n_shared] slot of each fat 4-bit expert's fp16 copies,
 *                -1 for the others (NULL without a fat route);
 *   fat_copy     the fp16 copies the dequantise-once step writes of the fat
 *                experts' W_gate, W_up and W_down (Strata PR #4366,
 *                "Approach": an expert's weights decoded to FP16 once): slot
 *                s of matrix m ([N, K] = [F, D], [F, D], [D, F]) starts
 *                s * N * K values after fat_copy[m] and is laid out
 *                [K / 32][N][32] (NULL without a fat route); fat_slots is
 *                the number of slots the workspace holds.
 * Returns MOE_EINVAL on a NULL plan, ws or out, or sizes the workspace query
 * refuses. */
typedef struct {
    const void *h, *h_lo;
    int64_t h_ld;
    const void *ht, *ht_lo;
    int64_t pairs_max;
    const void *ypair;
    int32_t ypair_dtype;
    const int32_t *fat_slot;
    const void *fat_copy[3];
    int64_t fat_slots;
} moe_forward_views;

moe_status moe_forward_get_views(const moe_plan *plan, int32_t D, int32_t F,
                                 int32_t x_dtype, int32_t w_dtype,
                                 const moe_options *opt, const void *ws,
                                 moe_forward_views *out);

/* --- backward ----------------------------------------------------------- */

/* Bytes of device workspace moe_backward needs; 0 if unsupported. */
size_t moe_backward_workspace_bytes(const moe_plan *plan, int32_t D, int32_t F,
                                    int32_t x_dtype);

/* Gradients of L = sum_t dy[t] . y[t] for the layer moe_forward computes on
 * the same plan, x and weights (bf16 or f16 layers: x and the three weights
 * in one 16-bit dtype; 4-bit weights are not trained here): dx [T, D],
 * dw_gate / dw_up [E + n_shared, F, D], dw_down [E + n_shared, D, F], all
 * f32 and overwritten; every expert slot gets the sum over its kept pairs
 * (zeros for an expert with none), the property mini-AGI PR #3's
 * tests/test_dispatch.py asks of every dispatch. Optional (NULL to skip):
 * d_topk_w [T, k], the gradient of each routing weight (dy[t] . the pair's
 * unweighted output; 0 for a dropped pair), and d_logits [T, E], through the
 * renormalised top-k softmax (w_j (dw_j - sum_i w_i dw_i) on the chosen
 * experts, 0 elsewhere). The expert outputs are recomputed from x (nothing
 * is kept from the forward); per-pair intermediates (x rows, dy rows, w
 * times the SwiGLU output, the SwiGLU gradients) are held in the layer's
 * dtype, products accumulate in f32. opt: the swiglu_limit of the forward
 * (NULL: defaults); MOE_OPT_PHASE_EVENTS times its four phases
 * (moe_phase_times 10..13; MOE_OPT_PHASE_ONLY bits select among them). D and F multiples of 128; pointers 16-byte
 * aligned, ws 256-byte aligned. MOE_EUNSUPPORTED when x, a per-pair operand
 * (T k + n_shared T pairs x max(2F, D) 16-bit values) or a weight matrix
 * reaches 2 GiB. Async on `stream`. */
moe_status moe_backward(const moe_plan *plan, const void *x, int32_t x_dtype,
                        moe_weight w_gate, moe_weight w_up, moe_weight w_down,
                        int32_t D, int32_t F, const float *dy, float *dx,
                        float *dw_gate, float *dw_up, float *dw_down,
                        float *d_topk_w, float *d_logits, void *ws,
                        size_t ws_bytes, const moe_options *opt, void *stream);

/* --- standalone pieces ------------------------------------------------- */

/* Dequantise rows of 4-bit block weights to fp16, once: out[r, c] =
 * fp16_rne(q * s) for a [rows, K] matrix (Strata PR #4366, "Approach": one
 * expert's weights decoded to FP16 once). K multiple of 32. Async. */
moe_status moe_dequant_q4(const void *data, const void *scales, int64_t rows,
                          int64_t K, void *out_f16, void *stream);

/* Dequantise rows of any 4-bit format (MOE_Q4B32, MOE_Q4A32, MOE_Q4A64) to
 * fp16 once: out[r, c] = fp16_rne(q * s) or fp16_rne(q * s + b) (one
 * rounding: the affine value is one fp16 fma). K a multiple of the group
 * (32 or 64); data and out 16-byte aligned, scales 2-byte (Q4B32) or
 * 4-byte (affine). Async. */
moe_status moe_dequant_weights(int32_t dtype, const void *data,
                               const void *scales, int64_t rows, int64_t K,
                               void *out_f16, void *stream);

/* Milliseconds spent in each phase, summed over the moe_forward and
 * moe_route calls since the last reset that ran with MOE_OPT_PHASE_EVENTS;
 * `calls` receives the number of such calls. Phases: 0 classify,
 * 1 dequant-once, 2 gate/up full tile, 3 gate/up split-K groups of <= 16
 * rows, 4 down full tile, 5 down split-K groups of <= 16 rows, 6 combine,
 * 14 gate/up split-K groups of 17..64 rows, 15 down groups of 17..64 rows
 * (moe_forward); 7 router kernel, 8 plan, 9 routing statistics
 * (moe_route); 10 recompute, 11 data gradients, 12 weight gradients,
 * 13 routing-weight gradients (moe_backward). Synchronises on the recorded
 * events. reset != 0 clears afterwards. */
#define MOE_N_PHASES 16
moe_status moe_phase_times(double *ms, int32_t n, int64_t *calls,
                           int32_t reset);

/* Thread-local message for the last non-OK status of this thread. */
const char *moe_last_error(void);

/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
