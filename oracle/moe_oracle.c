/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU oracle for the forward pass of a routed
 * mixture-of-experts FFN layer on a prompt. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the HIP library never
 * does, and the two share no code, header, table or helper.
 *
 * What it computes, and where the pages say so:
 *   route    top-k of the router over each token, the chosen weights
 *            renormalised to sum to one (mini-AGI PR #3, minagi/pool.py,
 *            `requested(scores)`, the comment on the kept mass).
 *   plan     capacity drop in token order: a pair is kept while its expert
 *            holds fewer than `limit` earlier pairs; pairs sorted by expert
 *            (mini-AGI PR #3 and #4, minagi/pool.py, the `keep` filter and the
 *            argsort/bincount over the flattened expert ids; the capacity
 *            factor caps an expert at a multiple of its even share of the
 *            batch, configs/strix_halo_large.yaml, `capacity_factor`).
 *   expert   h = silu(x Wg^T) * (x Wu^T), y = h Wd^T (mini-AGI PR #4,
 *            minagi/pool.py, `experts()`), with the clamp of the FP16 fat
 *            expert route (Strata PR #4366, "Problem and result" and
 *            "Approach").
 *   combine  y[t] = sum over kept pairs of weight * expert output; a dropped
 *            pair adds nothing (the weights are filtered by `keep` after they
 *            were normalised, mini-AGI PR #4, minagi/pool.py).
 *   backward gradients of the layer (x, the three expert weights, the
 *            routing weights and, through them, the logits): the same
 *            gradients on every expert slot whatever the dispatch (mini-AGI
 *            PR #3, tests/test_dispatch.py).
 *   router   logits = x Wr^T, the linear map from d_model to the experts
 *            whose output `requested(scores)` ranks, and the statistics that
 *            function keeps beside the routing: the top-k mass before
 *            renormalisation, the number of experts the router wants (the
 *            fewest holding 90 % of the softmax mass), and the auxiliary loss
 *            (balance term plus z-loss weighted by z_weight) (mini-AGI PR #3,
 *            minagi/pool.py, `requested(scores)` and the `__init__` signature
 *            with z_weight=1e-3).
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *   - top-k by logits (softmax is monotone), ties to the lower expert index,
 *     +0 and -0 equal; NaN logits are refused;
 *   - limit = max(1, floor(cf * T * k / E)); cf == 0 means no cap;
 *   - the clamp: gate clamped above at c, up clamped to [-c, c], c <= 0 off;
 *   - a shared expert (index E) sees every token with weight 1, never drops;
 *   - 4-bit weights: two's-complement nibbles, low nibble = even K index,
 *     one fp16 scale per 32 consecutive K values of an output row, value q*s;
 *     the affine 4-bit groups: unsigned nibbles (low nibble = even K index),
 *     an fp16 scale and bias per 32 or 64 K values stored as interleaved
 *     pairs, value q*s + b;
 *   - router statistics: `want` is counted per token (largest p first, the
 *     first count whose running sum is >= 0.9) and averaged over tokens; the
 *     balance term's first choice is rank 0 of the top-k rule above.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC moe_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2, ORC_Q4B32 = 3, ORC_Q4A32 = 4,
       ORC_Q4A64 = 5 };

static int is_q4(int dtype)
{
    return dtype == ORC_Q4B32 || dtype == ORC_Q4A32 || dtype == ORC_Q4A64;
}

/* K values that share one scale (and, for the affine formats, one bias). */
static int q4_group(int dtype)
{
    return dtype == ORC_Q4A64 ? 64 : 32;
}

/* ---- exact decoding of stored values ---------------------------------- */

/* IEEE 754 binary16 -> double, exact (sign, 5-bit exponent, 10-bit fraction). */
static double f16_bits_to_double(uint16_t h)
{
    int sign = h >> 15;
    int ex = (h >> 10) & 31;
    int fr = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);               /* subnormal: fr * 2^-24 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr + 1024), ex - 25);  /* (1 + fr/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double dense_value(const void *base, int dtype, size_t idx)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_BF16: return bf16_bits_to_double(((const uint16_t *)base)[idx]);
    case ORC_F16: return f16_bits_to_double(((const uint16_t *)base)[idx]);
    default: return NAN;
    }
}

/* Element (n, kk) of expert e's [N, K] weight matrix, decoded exactly.
 * Q4B32: two's-complement nibbles, value q * s, one fp16 scale per 32 K
 * values ([.., N, K/32]). Q4A32 / Q4A64: unsigned nibbles 0..15, value
 * q * s + b with an fp16 (scale, bias) pair per 32 / 64 K values, the pairs
 * interleaved ([.., N, K/G, 2]) -- the affine 4-bit groups of the MLX
 * checkpoints TensorFold PR #1607 serves (its tuner tables: "group 64",
 * "group 32"). q * s + b is exact in double (a 15-bit product plus an fp16). */
static double weight_value(const void *data, const void *scales, int dtype,
                           int64_t e, int64_t N, int64_t K, int64_t n, int64_t kk)
{
    if (!is_q4(dtype))
        return dense_value(data, dtype, (size_t)((e * N + n) * K + kk));
    const uint8_t *bytes = (const uint8_t *)data;
    uint8_t byte = bytes[(e * N + n) * (K / 2) + kk / 2];
    int nib = (kk & 1) ? (byte >> 4) : (byte & 15);
    const uint16_t *s = (const uint16_t *)scales;
    if (dtype == ORC_Q4B32) {
        int q = nib >= 8 ? nib - 16 : nib;       /* two's complement, -8..7 */
        double scale = f16_bits_to_double(s[(e * N + n) * (K / 32) + kk / 32]);
        return (double)q * scale;
    }
    int64_t G = q4_group(dtype);
    int64_t at = ((e * N + n) * (K / G) + kk / G) * 2;
    return (double)nib * f16_bits_to_double(s[at]) + f16_bits_to_double(s[at + 1]);
}

/* Decode one expert's [N, K] matrix into out (row-major), for the tests. */
int orc_decode(const void *data, const void *scales, int dtype, int64_t e,
               int64_t N, int64_t K, double *out)
{
    if (dtype < ORC_F32 || dtype > ORC_Q4A64 || (is_q4(dtype) && K % q4_group(dtype)))
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kk = 0; kk < K; ++kk)
            out[n * K + kk] = weight_value(data, scales, dtype, e, N, K, n, kk);
    return 0;
}

int orc_decode_f16(const uint16_t *bits, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_bits_to_double(bits[i]);
    return 0;
}

/* ---- route ------------------------------------------------------------- */

/*
 * For every token: the k experts of largest logit, ordered by rank, where the
 * rank of expert e is the number of experts that beat it (a larger logit, or
 * an equal logit and a lower index). Weights w_j = exp(l_j - l_0) / sum_i
 * exp(l_i - l_0) over the k chosen: full softmax renormalised over the top-k.
 */
int orc_route(int64_t T, int E, int k, const float *logits, int32_t *ids,
              double *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    for (int64_t i = 0; i < T * E; ++i)
        if (isnan(logits[i]))
            return -2;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        int found = 0;
        for (int e = 0; e < E; ++e) {
            int rank = 0;
            for (int f = 0; f < E; ++f)
                if (l[f] > l[e] || (l[f] == l[e] && f < e))
                    ++rank;
            if (rank < k) {
                ids[t * k + rank] = e;
                ++found;
            }
        }
        if (found != k) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double l0 = (double)l[ids[t * k]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += exp((double)l[ids[t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            w[t * k + j] = exp((double)l[ids[t * k + j]] - l0) / sum;
    }
    return bad ? -3 : 0;
}

/* ---- capacity and dispatch plan --------------------------------------- */

/* Most pairs one expert may keep: cf times its fair share T*k/E, floored,
 * at least 1; -1 means uncapped (cf == 0). */
int64_t orc_limit(int64_t T, int E, int k, double cf)
{
    if (cf == 0.0)
        return -1;
    double fair = cf * (double)T * (double)k / (double)E;
    int64_t lim = (int64_t)floor(fair);
    return lim < 1 ? 1 : lim;
}

/*
 * Walk the pairs in token order. slot = how many earlier tokens chose the
 * same expert; keep iff slot < limit. Kept pairs are placed in an
 * expert-sorted list at offsets[e] + slot. The shared expert, when present, is
 * index E and holds every token in order, weight 1, never dropped.
 * Outputs (caller-allocated): slot[T*k], keep[T*k], counts[E+ns],
 * offsets[E+ns+1], pair_token[P], pair_src[P] (t*k+j, or -1 for a shared
 * pair), tok2pair[T*k] (-1 when dropped), *dropped, *limit_out.
 */
int orc_plan(int64_t T, int E, int k, int n_shared, double cf,
             const int32_t *ids, int64_t *limit_out, int32_t *slot,
             uint8_t *keep, int64_t *counts, int64_t *offsets,
             int32_t *pair_token, int32_t *pair_src, int32_t *tok2pair,
             int64_t *dropped)
{
    if (T < 0 || E < 1 || k < 1 || k > E || n_shared < 0 || n_shared > 1 ||
        !(cf >= 0.0) || isinf(cf))
        return -1;
    int64_t limit = orc_limit(T, E, k, cf);
    int64_t *seen = calloc((size_t)E, sizeof *seen);
    if (!seen)
        return -4;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = ids[t * k + j];
            if (e < 0 || e >= E) {
                free(seen);
                return -1;
            }
            int64_t s = seen[e]++;
            slot[t * k + j] = (int32_t)s;
            keep[t * k + j] = (limit < 0 || s < limit) ? 1 : 0;
        }
    int64_t kept = 0;
    for (int e = 0; e < E; ++e) {
        counts[e] = (limit < 0 || seen[e] < limit) ? seen[e] : limit;
        kept += counts[e];
    }
    if (n_shared)
        counts[E] = T;
    offsets[0] = 0;
    for (int e = 0; e < E + n_shared; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t p = t * k + j;
            if (keep[p]) {
                int64_t pos = offsets[ids[p]] + slot[p];
                pair_token[pos] = (int32_t)t;
                pair_src[pos] = (int32_t)p;
                tok2pair[p] = (int32_t)pos;
            } else {
                tok2pair[p] = -1;
            }
        }
    if (n_shared)
        for (int64_t t = 0; t < T; ++t) {
            pair_token[offsets[E] + t] = (int32_t)t;
            pair_src[offsets[E] + t] = -1;
        }
    *dropped = T * k - kept;
    *limit_out = limit;
    free(seen);
    return 0;
}

/* ---- one expert on one token ------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * g = Wg[e] x, u = Wu[e] x, h = silu(min(g, c)) * clamp(u, -c, c) (no clamp
 * when c <= 0), yp = Wd[e] h. Any of g, u, h, yp may be NULL. par != 0
 * spreads the independent rows over OpenMP threads (for a caller outside a
 * parallel region); each value is computed the same way either way.
 */
static void expert_ffn(int64_t D, int64_t F, int64_t e, const double *x,
                       const void *wg, const void *wg_s, const void *wu,
                       const void *wu_s, const void *wd, const void *wd_s,
                       int w_dtype, double c, double *g, double *u, double *h,
                       double *yp, int par)
{
    double *hh = malloc((size_t)F * sizeof *hh);
#pragma omp parallel for schedule(static) if (par)
    for (int64_t f = 0; f < F; ++f) {
        double gs = 0.0, us = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            gs += weight_value(wg, wg_s, w_dtype, e, F, D, f, d) * x[d];
            us += weight_value(wu, wu_s, w_dtype, e, F, D, f, d) * x[d];
        }
        double gc = gs, uc = us;
        if (c > 0.0) {
            gc = gs < c ? gs : c;
            uc = us < -c ? -c : (us > c ? c : us);
        }
        hh[f] = silu(gc) * uc;
        if (g) g[f] = gs;
        if (u) u[f] = us;
        if (h) h[f] = hh[f];
    }
#pragma omp parallel for schedule(static) if (par && yp)
    for (int64_t d = 0; d < (yp ? D : 0); ++d) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f)
            s += weight_value(wd, wd_s, w_dtype, e, D, F, d, f) * hh[f];
        yp[d] = s;
    }
    free(hh);
}

int orc_expert(int64_t D, int64_t F, int64_t e, const void *xrow, int x_dtype,
               const void *wg, const void *wg_s, const void *wu,
               const void *wu_s, const void *wd, const void *wd_s,
               int w_dtype, double c, double *g, double *u, double *h,
               double *yp)
{
    if (x_dtype < ORC_F32 || x_dtype > ORC_F16 || w_dtype < ORC_F32 ||
        w_dtype > ORC_Q4A64)
        return -1;
    double *x = malloc((size_t)D * sizeof *x);
    for (int64_t d = 0; d < D; ++d)
        x[d] = dense_value(xrow, x_dtype, (size_t)d);
    expert_ffn(D, F, e, x, wg, wg_s, wu, wu_s, wd, wd_s, w_dtype, c, g, u, h,
               yp, 0);
    free(x);
    return 0;
}

/*
 * The unweighted expert output of n (token, expert) pairs, yp[i] =
 * FFN_{experts[i]}(x[tokens[i]]): the rows the combine weighs and sums
 * (mini-AGI PR #4, minagi/pool.py, `experts()` then the weighted gather
 * back to tokens). One pair per OpenMP iteration.
 */
int orc_pairs(int64_t n, int64_t T, int64_t D, int64_t F, int n_exp,
              const int64_t *tokens, const int32_t *experts, const void *x,
              int x_dtype, const void *wg, const void *wg_s, const void *wu,
              const void *wu_s, const void *wd, const void *wd_s,
              int w_dtype, double c, double *yp)
{
    if (x_dtype < ORC_F32 || x_dtype > ORC_F16 || w_dtype < ORC_F32 ||
        w_dtype > ORC_Q4A64 ||
        (is_q4(w_dtype) && (D % q4_group(w_dtype) || F % q4_group(w_dtype))))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= T || experts[i] < 0 ||
            experts[i] >= n_exp)
            return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        double *xt = malloc((size_t)D * sizeof *xt);
        for (int64_t d = 0; d < D; ++d)
            xt[d] = dense_value(x, x_dtype, (size_t)(tokens[i] * D + d));
        expert_ffn(D, F, experts[i], xt, wg, wg_s, wu, wu_s, wd, wd_s,
                   w_dtype, c, NULL, NULL, NULL, yp + i * D, 0);
        free(xt);
    }
    return 0;
}

/* ---- the layer --------------------------------------------------------- */

/*
 * y[t] = sum_j keep[t,j] * w[t,j] * expert(ids[t,j], x[t]) (+ shared expert),
 * for the tokens in tok_list (all T tokens when tok_list is NULL). No
 * renormalisation after drops.
 */
int orc_layer(int64_t T, int64_t D, int64_t F, int E, int k, int n_shared,
              const void *x, int x_dtype, const void *wg, const void *wg_s,
              const void *wu, const void *wu_s, const void *wd,
              const void *wd_s, int w_dtype, double c, const int32_t *ids,
              const double *w, const uint8_t *keep, int64_t n_tok,
              const int64_t *tok_list, double *y)
{
    if (x_dtype < ORC_F32 || x_dtype > ORC_F16 || w_dtype < ORC_F32 ||
        w_dtype > ORC_Q4A64 ||
        (is_q4(w_dtype) && (D % q4_group(w_dtype) || F % q4_group(w_dtype))))
        return -1;
    if (!tok_list)
        n_tok = T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tok; ++i) {
        int64_t t = tok_list ? tok_list[i] : i;
        double *xt = malloc((size_t)D * sizeof *xt);
        double *yp = malloc((size_t)D * sizeof *yp);
        double *yt = y + i * D;
        for (int64_t d = 0; d < D; ++d) {
            xt[d] = dense_value(x, x_dtype, (size_t)(t * D + d));
            yt[d] = 0.0;
        }
        for (int j = 0; j < k; ++j) {
            if (!keep[t * k + j])
                continue;
            expert_ffn(D, F, ids[t * k + j], xt, wg, wg_s, wu, wu_s, wd, wd_s,
                       w_dtype, c, NULL, NULL, NULL, yp, 0);
            for (int64_t d = 0; d < D; ++d)
                yt[d] += w[t * k + j] * yp[d];
        }
        if (n_shared) {
            expert_ffn(D, F, E, xt, wg, wg_s, wu, wu_s, wd, wd_s, w_dtype, c,
                       NULL, NULL, NULL, yp, 0);
            for (int64_t d = 0; d < D; ++d)
                yt[d] += yp[d];
        }
        free(xt);
        free(yp);
    }
    return 0;
}

/* ---- backward ---------------------------------------------------------- */

/*
 * Gradients of L = sum_t dy[t] . y[t] for one kept pair (token row x, expert
 * e) whose output is scaled by its weight: dyp = weight * dy[t]. The layer's
 * forward is y[t] = sum_j keep * w_j * FFN_e(x[t]) (+ the shared expert's
 * FFN), FFN_e(x) = W_down h, h = silu(min(g, c)) * clamp(u, -c, c),
 * g = W_gate x, u = W_up x (mini-AGI PR #4, minagi/pool.py, `experts()`;
 * the clamp of Strata PR #4366, "Approach"). The clamps pass the gradient
 * where the value is not clamped, boundaries included (g <= c, -c <= u <=
 * c), like a clamp's subgradient in autograd. Accumulates into dx (D),
 * dwg / dwu (F x D), dwd (D x F) when they are not NULL. par != 0 (only
 * with dx NULL: its sum runs over f) spreads the rows f over OpenMP
 * threads, each row computed the same way.
 */
static void pair_backward(int64_t D, int64_t F, int64_t e, const double *x,
                          const void *wg, const void *wg_s, const void *wu,
                          const void *wu_s, const void *wd, const void *wd_s,
                          int w_dtype, double c, const double *dyp, double *dx,
                          double *dwg, double *dwu, double *dwd, int par)
{
    double *g = malloc((size_t)F * sizeof *g);
    double *u = malloc((size_t)F * sizeof *u);
    double *h = malloc((size_t)F * sizeof *h);
    expert_ffn(D, F, e, x, wg, wg_s, wu, wu_s, wd, wd_s, w_dtype, c, g, u, h,
               NULL, par);
#pragma omp parallel for schedule(static) if (par && !dx)
    for (int64_t f = 0; f < F; ++f) {
        double dh = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dh += weight_value(wd, wd_s, w_dtype, e, D, F, d, f) * dyp[d];
        double gc = g[f], uc = u[f], mg = 1.0, mu = 1.0;
        if (c > 0.0) {
            if (g[f] > c) { gc = c; mg = 0.0; }
            if (u[f] < -c) { uc = -c; mu = 0.0; }
            if (u[f] > c) { uc = c; mu = 0.0; }
        }
        double sg = 1.0 / (1.0 + exp(-gc));
        double dsilu = sg * (1.0 + gc * (1.0 - sg));
        double dg = dh * uc * dsilu * mg;
        double du = dh * gc * sg * mu;
        for (int64_t d = 0; d < D; ++d) {
            double wgv = weight_value(wg, wg_s, w_dtype, e, F, D, f, d);
            double wuv = weight_value(wu, wu_s, w_dtype, e, F, D, f, d);
            if (dx)
                dx[d] += wgv * dg + wuv * du;
            if (dwg)
                dwg[f * D + d] += dg * x[d];
            if (dwu)
                dwu[f * D + d] += du * x[d];
        }
        if (dwd)
            for (int64_t d = 0; d < D; ++d)
                dwd[d * F + f] += dyp[d] * h[f];
    }
    free(g); free(u); free(h);
}

/*
 * Backward of the layer for L = sum_t dy[t] . y[t] (dy [T, D] double):
 *   dx   [n_tok, D]        for the tokens of tok_list (all T if NULL);
 *   dwg, dwu [n_exp, F, D] and dwd [n_exp, D, F] for the experts of
 *        exp_list (all E + n_shared if NULL; index E is the shared one);
 *   dtw  [T, k]            gradient of each routing weight w_j: dy[t] .
 *        FFN(x[t]) for a kept pair, 0 for a dropped one (NULL: skipped).
 * Gradients of the expert weights are the sums over the expert's kept pairs
 * -- mini-AGI PR #3's tests/test_dispatch.py asks any dispatch to give each
 * expert slot the gradient running every expert gives. Any pointer may be
 * NULL.
 */
int orc_backward(int64_t T, int64_t D, int64_t F, int E, int k, int n_shared,
                 const void *x, int x_dtype, const void *wg, const void *wg_s,
                 const void *wu, const void *wu_s, const void *wd,
                 const void *wd_s, int w_dtype, double c, const int32_t *ids,
                 const double *w, const uint8_t *keep, const double *dy,
                 int64_t n_tok, const int64_t *tok_list, double *dx,
                 int n_exp, const int32_t *exp_list, double *dwg, double *dwu,
                 double *dwd, double *dtw)
{
    if (x_dtype < ORC_F32 || x_dtype > ORC_F16 || w_dtype < ORC_F32 ||
        w_dtype > ORC_Q4A64)
        return -1;
    if (!tok_list)
        n_tok = T;
    if (!exp_list)
        n_exp = E + n_shared;
    if (dx) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_tok; ++i) {
            int64_t t = tok_list ? tok_list[i] : i;
            double *xt = malloc((size_t)D * sizeof *xt);
            double *dyp = malloc((size_t)D * sizeof *dyp);
            double *dxt = dx + i * D;
            for (int64_t d = 0; d < D; ++d) {
                xt[d] = dense_value(x, x_dtype, (size_t)(t * D + d));
                dxt[d] = 0.0;
            }
            for (int j = 0; j <= k; ++j) {
                int64_t e;
                double wt;
                if (j < k) {
                    if (!keep[t * k + j])
                        continue;
                    e = ids[t * k + j];
                    wt = w[t * k + j];
                } else {
                    if (!n_shared)
                        break;
                    e = E;
                    wt = 1.0;
                }
                for (int64_t d = 0; d < D; ++d)
                    dyp[d] = wt * dy[t * D + d];
                pair_backward(D, F, e, xt, wg, wg_s, wu, wu_s, wd, wd_s, w_dtype,
                              c, dyp, dxt, NULL, NULL, NULL, 0);
            }
            free(xt); free(dyp);
        }
    }
    if (dwg || dwu || dwd) {
        /* one expert, one kept pair at a time, in token order; the rows f of
         * a pair's gradient are spread over the threads (an expert may hold
         * most of the pairs) */
        for (int i = 0; i < n_exp; ++i) {
            int64_t e = exp_list ? exp_list[i] : i;
            double *xt = malloc((size_t)D * sizeof *xt);
            double *dyp = malloc((size_t)D * sizeof *dyp);
            double *g_ = dwg ? dwg + (size_t)i * F * D : NULL;
            double *u_ = dwu ? dwu + (size_t)i * F * D : NULL;
            double *d_ = dwd ? dwd + (size_t)i * D * F : NULL;
            if (g_) memset(g_, 0, (size_t)F * D * sizeof *g_);
            if (u_) memset(u_, 0, (size_t)F * D * sizeof *u_);
            if (d_) memset(d_, 0, (size_t)D * F * sizeof *d_);
            for (int64_t t = 0; t < T; ++t) {
                double wt = 0.0;
                int hit = 0;
                if (e == E) {
                    hit = n_shared;
                    wt = 1.0;
                } else {
                    for (int j = 0; j < k; ++j)
                        if (ids[t * k + j] == e && keep[t * k + j]) {
                            hit = 1;
                            wt = w[t * k + j];
                        }
                }
                if (!hit)
                    continue;
                for (int64_t d = 0; d < D; ++d) {
                    xt[d] = dense_value(x, x_dtype, (size_t)(t * D + d));
                    dyp[d] = wt * dy[t * D + d];
                }
                pair_backward(D, F, e, xt, wg, wg_s, wu, wu_s, wd, wd_s, w_dtype,
                              c, dyp, NULL, g_, u_, d_, 1);
            }
            free(xt); free(dyp);
        }
    }
    if (dtw) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            double *xt = malloc((size_t)D * sizeof *xt);
            double *yp = malloc((size_t)D * sizeof *yp);
            for (int64_t d = 0; d < D; ++d)
                xt[d] = dense_value(x, x_dtype, (size_t)(t * D + d));
            for (int j = 0; j < k; ++j) {
                double s = 0.0;
                if (keep[t * k + j]) {
                    expert_ffn(D, F, ids[t * k + j], xt, wg, wg_s, wu, wu_s, wd,
                               wd_s, w_dtype, c, NULL, NULL, NULL, yp, 0);
                    for (int64_t d = 0; d < D; ++d)
                        s += dy[t * D + d] * yp[d];
                }
                dtw[t * k + j] = s;
            }
            free(xt); free(yp);
        }
    }
    return 0;
}

/*
 * Gradient of the logits through the chosen weights w_j = exp(l_j - l_0) /
 * sum_i exp(l_i - l_0) (softmax renormalised over the k chosen): dl[t, e_j]
 * = w_j (dtw_j - sum_i w_i dtw_i); experts not chosen get 0 (the top-k
 * choice is constant under small changes of the logits). out [T, E].
 */
int orc_dlogits(int64_t T, int E, int k, const int32_t *ids, const double *w,
                const double *dtw, double *out)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j)
            s += w[t * k + j] * dtw[t * k + j];
        for (int e = 0; e < E; ++e)
            out[t * E + e] = 0.0;
        for (int j = 0; j < k; ++j)
            out[t * E + ids[t * k + j]] = w[t * k + j] * (dtw[t * k + j] - s);
    }
    return 0;
}

/* ---- router logits and routing statistics ------------------------------ */

/*
 * logits[t, e] = sum_d x[t, d] * Wr[e, d], in double over the exactly decoded
 * inputs (x [T, D] and Wr [E, D] of one dense dtype). The pages route the
 * output of this map (mini-AGI PR #3, minagi/pool.py, `requested(scores)`).
 */
int orc_router_logits(int64_t T, int64_t D, int E, const void *x, int dtype,
                      const void *wr, double *out)
{
    if (T < 0 || D < 1 || E < 1 || dtype < ORC_F32 || dtype > ORC_F16)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t d = 0; d < D; ++d)
                s += dense_value(x, dtype, (size_t)(t * D + d)) *
                     dense_value(wr, dtype, (size_t)((int64_t)e * D + d));
            out[t * E + e] = s;
        }
    return 0;
}

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/*
 * Statistics of one routing call over the logits it ranked (mini-AGI PR #3,
 * minagi/pool.py, `requested(scores)`), each token's p = softmax of its E
 * logits:
 *   out[0] kept mass: mean over tokens of the mass of p on the k chosen
 *          experts, taken before the k weights are renormalised;
 *   out[1] want_k: mean over tokens of the fewest experts whose p, largest
 *          first, add up to at least 0.9 (want_t[t] per token);
 *   out[2] z loss: mean over tokens of logsumexp(logits[t])^2;
 *   out[3] balance: E * sum_e frac_e * mean_t p[t, e], frac_e = share of the
 *          tokens whose first choice is e;
 *   out[4] aux = balance + z_weight * z loss.
 * The chosen experts and the first choice follow orc_route's rank rule.
 * T == 0 gives zeros. NaN logits: -2.
 */
int orc_router_stats(int64_t T, int E, int k, const float *logits,
                     double z_weight, double *out, int32_t *want_t)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    for (int i = 0; i < 5; ++i)
        out[i] = 0.0;
    if (T == 0)
        return 0;
    int32_t *ids = malloc((size_t)T * k * sizeof *ids);
    double *w = malloc((size_t)T * k * sizeof *w);
    double *p = malloc((size_t)T * E * sizeof *p);
    double *kept = malloc((size_t)T * sizeof *kept);
    double *z = malloc((size_t)T * sizeof *z);
    int32_t *need = want_t ? want_t : malloc((size_t)T * sizeof *need);
    if (!ids || !w || !p || !kept || !z || !need) {
        free(ids); free(w); free(p); free(kept); free(z);
        if (!want_t)
            free(need);
        return -4;
    }
    int rc = orc_route(T, E, k, logits, ids, w);
    if (rc == 0) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float *l = logits + t * E;
            double *pt = p + t * E;
            double m = (double)l[0];
            for (int e = 1; e < E; ++e)
                if ((double)l[e] > m)
                    m = (double)l[e];
            double s = 0.0;
            for (int e = 0; e < E; ++e)
                s += exp((double)l[e] - m);
            for (int e = 0; e < E; ++e)
                pt[e] = exp((double)l[e] - m) / s;
            double lse = m + log(s);
            z[t] = lse * lse;
            double km = 0.0;
            for (int j = 0; j < k; ++j)
                km += pt[ids[t * k + j]];
            kept[t] = km;
            double *sorted = malloc((size_t)E * sizeof *sorted);
            memcpy(sorted, pt, (size_t)E * sizeof *sorted);
            qsort(sorted, (size_t)E, sizeof *sorted, cmp_desc);
            double run = 0.0;
            int m_need = E;
            for (int i = 0; i < E; ++i) {
                run += sorted[i];
                if (run >= 0.9) {
                    m_need = i + 1;
                    break;
                }
            }
            free(sorted);
            need[t] = m_need;
        }
        double sk = 0.0, sw = 0.0, sz = 0.0, bal = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            sk += kept[t];
            sw += (double)need[t];
            sz += z[t];
        }
        for (int e = 0; e < E; ++e) {
            double mp = 0.0;
            int64_t first = 0;
            for (int64_t t = 0; t < T; ++t) {
                mp += p[t * E + e];
                first += ids[t * k] == e;
            }
            bal += ((double)first / (double)T) * (mp / (double)T);
        }
        out[0] = sk / (double)T;
        out[1] = sw / (double)T;
        out[2] = sz / (double)T;
        out[3] = (double)E * bal;
        out[4] = out[3] + z_weight * out[2];
    }
    free(ids); free(w); free(p); free(kept); free(z);
    if (!want_t)
        free(need);
    return rc;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
