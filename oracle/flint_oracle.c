/*
 * flint_oracle.c -- plain, slow CPU oracle for the Flint routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU path is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  The product library never links, loads or calls it,
 * and it shares no code, header or table with the GPU path.
 *
 * What it computes (sources are the pages on the Flint release):
 *   - "Recursive Flint serving kit" review, section "The architecture, from the
 *     config": 256 routed experts per MoE layer, 6 selected per token, plus an
 *     always-on shared expert; expert intermediate size 512, shared expert 1024;
 *     router scores are sigmoids and the top-k scores are renormalised (not a
 *     softmax).
 *   - "Recursive opens Flint, a 40B coding model with 2.5B active", section
 *     "What runs on each token": a router picks 6 of 256 expert sub-networks for
 *     each token and one shared expert runs every time.
 *   - The parameter count in the serving-kit review (routed experts about 37.8B,
 *     six experts plus the shared expert about 1.2B per token over 47 layers)
 *     selects the gated three-matrix form of each expert:
 *         expert(x) = W_down . ( silu(W_gate x) * (W_up x) ),  silu(g) = g*sigmoid(g).
 *
 * Arithmetic: every dot product and every intermediate is IEEE double.  Inputs
 * arrive as float arrays holding the exact values of the layer's storage type
 * (bf16 values widen to float exactly).  The only narrowing steps are those the
 * layer definition itself has (the readings of the pages are listed with each
 * function):
 *   - the router logit and the sigmoid score are stored as float32 values, and
 *     selection compares those float32 scores;
 *   - the routing weight is stored as float32;
 *   - the gated intermediate h is stored in the layer's dtype (bf16 rounding,
 *     round-to-nearest-even, or float32);
 *   - the layer output is float32.
 *
 * No blocking, no fusion, no reordering: each loop is the definition written out.
 * OpenMP, when enabled, only splits the outer loop over tokens; every token's
 * arithmetic is independent of the others and runs in the same order.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int hidden;        /* H */
    int n_experts;     /* E */
    int top_k;         /* K */
    int inter;         /* I  (routed expert width) */
    int shared_inter;  /* Is (shared expert width; 0 = no shared expert) */
    int h_is_bf16;     /* 1: h is stored as bf16; 0: h is stored as float32 */
} oracle_dims;

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* ------------------------------------------------------------------------ */
/* Rounding helpers (own implementations, from the definitions of the formats) */

/* Round a double to the nearest bf16 value (8 significand bits), ties to even.
 * Written from the format's definition: find the binade with frexp, scale so
 * that one bf16 unit in the last place is 1.0, round with rint (the default
 * floating-point environment rounds half to even), scale back.  Subnormal bf16
 * values share float32's minimum exponent (-126), so the unit never drops
 * below 2^-133. */
static double round_bf16(double a)
{
    if (a == 0.0 || !isfinite(a)) return a;
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, 0.5 <= |m| < 1 */
    int ulp_exp = ex - 8;          /* 8 significand bits */
    if (ulp_exp < -133) ulp_exp = -133;
    double q = rint(ldexp(a, -ulp_exp));
    return ldexp(q, ulp_exp);
}

static double round_f32(double a) { return (double)(float)a; }

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Routing weight of a selected expert: its score over the sum of the selected
 * scores, as float32.  Every selected float32 score is zero only when every
 * logit lies below about -103.3 (the sigmoid then underflows float32); the
 * quotient is 0/0 there, and each selected expert gets the equal share 1/K,
 * which is what equal scores give. */
static float weight_of(double s, double sum, int K)
{
    if (sum > 0.0) return (float)(s / sum);
    return (float)(1.0 / K);
}

/* ------------------------------------------------------------------------ */
/* Router: logits, sigmoid scores, top-K selection, renormalised weights.
 *
 * Source: serving-kit review, "The architecture, from the config" (sigmoid
 * scoring, normalised top-k, not softmax) and the release news page, "What runs
 * on each token" (6 of 256 experts per token).
 * Readings:
 *   - logit z_e = float32( sum_h x[h]*Wr[e][h] + b_e ), the sum exact in double;
 *   - score s_e = float32( 1 / (1 + exp(-z_e)) );
 *   - selection: order experts by (s descending, e ascending) and keep the
 *     first K; equal float32 scores go to the lower expert index;
 *   - weights w_e = float32( s_e / sum_{j in S} s_j ) -- no scaling factor, no
 *     epsilon; 1/K each when every selected score is zero (weight_of);
 *   - output order of the selected set: ascending expert index;
 *   - near-tie flag: s_(K) - s_(K+1) < 1e-5 in that ordering (false if K == E).
 */
static void route_one(const oracle_dims *d, const float *x, const float *wr,
                      const float *bias, float *scores, int *sel_out,
                      float *w_out, unsigned char *tie_out)
{
    const int H = d->hidden, E = d->n_experts, K = d->top_k;
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += (double)x[h] * (double)wr[(size_t)e * H + h];
        if (bias) acc += (double)bias[e];
        float z = (float)acc;
        scores[e] = (float)sigmoid((double)z);
    }
    /* Selection by repeated scans: the k-th pick is the best expert not yet
     * picked, "best" meaning higher score, or equal score and lower index. */
    unsigned char taken[4096];
    memset(taken, 0, (size_t)E);
    int picked[64];
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || scores[e] > scores[best]) best = e;  /* strict '>' keeps the lower index on ties */
        }
        taken[best] = 1;
        picked[k] = best;
    }
    if (tie_out) {
        unsigned char tie = 0;
        if (K < E) {
            int next = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (next < 0 || scores[e] > scores[next]) next = e;
            }
            double gap = (double)scores[picked[K - 1]] - (double)scores[next];
            tie = gap < 1e-5;
        }
        *tie_out = tie;
    }
    /* Ascending expert order for the output set. */
    int n = 0;
    for (int e = 0; e < E; ++e)
        if (taken[e]) sel_out[n++] = e;
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += (double)scores[sel_out[k]];
    for (int k = 0; k < K; ++k) w_out[k] = weight_of((double)scores[sel_out[k]], sum, K);
}

static int check_dims(const oracle_dims *d)
{
    if (!d) return 0;
    if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->inter <= 0) return 0;
    if (d->top_k > d->n_experts || d->top_k > 64 || d->n_experts > 4096) return 0;
    if (d->shared_inter < 0) return 0;
    return 1;
}

int oracle_route(const oracle_dims *d, int T, const float *x, const float *wr,
                 const float *bias, int *topk_idx, float *topk_w,
                 unsigned char *near_tie)
{
    if (!check_dims(d) || T < 0 || (T > 0 && (!x || !wr || !topk_idx || !topk_w)))
        return ORACLE_BAD_ARG;
    const int H = d->hidden, K = d->top_k;
#pragma omp parallel for schedule(dynamic, 16)
    for (int t = 0; t < T; ++t) {
        float scores[4096];
        route_one(d, x + (size_t)t * H, wr, bias, scores, topk_idx + (size_t)t * K,
                  topk_w + (size_t)t * K, near_tie ? near_tie + t : NULL);
    }
    return ORACLE_OK;
}

/* Sigmoid scores only (float32 values as defined above), [T][E]. */
int oracle_scores(const oracle_dims *d, int T, const float *x, const float *wr,
                  const float *bias, float *scores)
{
    if (!check_dims(d) || T < 0 || (T > 0 && (!x || !wr || !scores))) return ORACLE_BAD_ARG;
    const int H = d->hidden, E = d->n_experts;
#pragma omp parallel for schedule(dynamic, 16)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)x[(size_t)t * H + h] * (double)wr[(size_t)e * H + h];
            if (bias) acc += (double)bias[e];
            float z = (float)acc;
            scores[(size_t)t * E + e] = (float)sigmoid((double)z);
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Dispatch: the token -> expert assignment regrouped by expert.
 *
 * Source: release news page, "What runs on each token" (a router picks 6 of 256
 * expert sub-networks for each token).  The grouping itself is a plain counting
 * sort, written as its definition:
 *   counts[e]      = number of tokens whose selected set contains e;
 *   offsets[e]     = counts[0] + ... + counts[e-1], offsets[E] = T*K;
 *   sorted_token   = for e = 0..E-1, then t ascending, every t with e in S_t;
 *   slot_of[t*K+k] = the position in sorted_token of the pair (t, topk_idx[t][k]).
 */
int oracle_dispatch(const oracle_dims *d, int T, const int *topk_idx, int *counts,
                    int *offsets, int *sorted_token, int *slot_of)
{
    if (!check_dims(d) || T < 0 || !counts || !offsets) return ORACLE_BAD_ARG;
    const int E = d->n_experts, K = d->top_k;
    if (T > 0 && (!topk_idx || !sorted_token || !slot_of)) return ORACLE_BAD_ARG;
    for (int i = 0; i < T * K; ++i)
        if (topk_idx[i] < 0 || topk_idx[i] >= E) return ORACLE_BAD_ARG;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int i = 0; i < T * K; ++i) counts[topk_idx[i]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int pos = 0;
    for (int e = 0; e < E; ++e)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                if (topk_idx[(size_t)t * K + k] == e) {
                    sorted_token[pos] = t;
                    slot_of[(size_t)t * K + k] = pos;
                    ++pos;
                }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* One gated expert applied to one token.
 *
 * Source: serving-kit review, "The architecture, from the config" (widths 512 and
 * 1024); the three-matrix gated form is the one the same page's parameter count
 * supports.  Reading: silu(g) = g * sigmoid(g), h = silu(g) * u stored in the
 * layer's dtype, y = W_down h.  Layouts: gate/up [width][H], down [H][width].
 */
static void expert_one(const oracle_dims *d, int width, const float *x,
                       const float *wg, const float *wu, const float *wd,
                       double *h_scratch, double *y)
{
    const int H = d->hidden;
    for (int i = 0; i < width; ++i) {
        double g = 0.0, u = 0.0;
        for (int k = 0; k < H; ++k) {
            g += (double)wg[(size_t)i * H + k] * (double)x[k];
            u += (double)wu[(size_t)i * H + k] * (double)x[k];
        }
        double a = g * sigmoid(g) * u;
        h_scratch[i] = d->h_is_bf16 ? round_bf16(a) : round_f32(a);
    }
    for (int n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int i = 0; i < width; ++i) acc += (double)wd[(size_t)n * width + i] * h_scratch[i];
        y[n] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* The whole layer for T tokens.
 *
 * out[t] = float32( sum_{e in S_t} w_e * expert_e(x_t) + shared(x_t) )
 *
 * Sources: serving-kit review, "The architecture, from the config" and release
 * news page, "What runs on each token".  Readings: the shared expert is added
 * with coefficient 1 (no gate); shared_inter == 0 means there is no shared
 * expert.
 *
 * force_idx (nullable, [T][K]): when given, use these expert sets instead of
 * the oracle's own selection; the weights are still this oracle's float32 scores
 * renormalised over the given set.  Used to check tokens whose K-th and (K+1)-th
 * scores are closer than the near-tie threshold, where either set is correct.
 * topk_idx_out, topk_w_out, near_tie (nullable) receive the routing used.
 */
int oracle_forward(const oracle_dims *d, int T, const float *x, const float *wr,
                   const float *bias, const float *wg, const float *wu, const float *wd,
                   const float *wsg, const float *wsu, const float *wsd,
                   const int *force_idx, float *out, int *topk_idx_out,
                   float *topk_w_out, unsigned char *near_tie)
{
    if (!check_dims(d) || T < 0) return ORACLE_BAD_ARG;
    if (T == 0) return ORACLE_OK;
    if (!x || !wr || !wg || !wu || !wd || !out) return ORACLE_BAD_ARG;
    if (d->shared_inter > 0 && (!wsg || !wsu || !wsd)) return ORACLE_BAD_ARG;
    const int H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter;
    if (force_idx)
        for (int i = 0; i < T * K; ++i)
            if (force_idx[i] < 0 || force_idx[i] >= E) return ORACLE_BAD_ARG;
    int bad = 0;
    const int wmax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        float scores[4096];
        int sel[64];
        float w[64];
        double *hbuf = (double *)malloc(sizeof(double) * (size_t)wmax);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        double *acc = (double *)malloc(sizeof(double) * (size_t)H);
        if (!hbuf || !y || !acc) {
#pragma omp atomic write
            bad = 1;
        } else {
            const float *xt = x + (size_t)t * H;
            unsigned char tie = 0;
            route_one(d, xt, wr, bias, scores, sel, w, &tie);
            if (force_idx) {
                double sum = 0.0;
                for (int k = 0; k < K; ++k) {
                    sel[k] = force_idx[(size_t)t * K + k];
                    sum += (double)scores[sel[k]];
                }
                for (int k = 0; k < K; ++k) w[k] = weight_of((double)scores[sel[k]], sum, K);
            }
            for (int n = 0; n < H; ++n) acc[n] = 0.0;
            for (int k = 0; k < K; ++k) {
                const int e = sel[k];
                expert_one(d, I, xt, wg + (size_t)e * I * H, wu + (size_t)e * I * H,
                           wd + (size_t)e * H * I, hbuf, y);
                for (int n = 0; n < H; ++n) acc[n] += (double)w[k] * y[n];
            }
            if (Is > 0) {
                expert_one(d, Is, xt, wsg, wsu, wsd, hbuf, y);
                for (int n = 0; n < H; ++n) acc[n] += y[n];
            }
            for (int n = 0; n < H; ++n) out[(size_t)t * H + n] = (float)acc[n];
            if (topk_idx_out)
                for (int k = 0; k < K; ++k) topk_idx_out[(size_t)t * K + k] = sel[k];
            if (topk_w_out)
                for (int k = 0; k < K; ++k) topk_w_out[(size_t)t * K + k] = w[k];
            if (near_tie) near_tie[t] = tie;
        }
        free(hbuf);
        free(y);
        free(acc);
    }
    return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* A dense MLP layer for T tokens (the model's first two layers are dense MLPs,
 * about 75M parameters together; serving-kit review, "The architecture, from
 * the config").  Reading: the same gated three-matrix form as an expert, of
 * width I (6144 fits the page's count: 2 * 3 * 2048 * 6144 = 75.5M), h stored
 * in the layer's dtype, out[t] = float32(W_down (silu(W_gate x_t) * (W_up x_t))).
 * Layouts: gate/up [I][H], down [H][I]. */
int oracle_dense_mlp(int T, int H, int I, int h_is_bf16, const float *x, const float *wg, const float *wu,
                     const float *wd, float *out)
{
    if (T < 0 || H <= 0 || I <= 0) return ORACLE_BAD_ARG;
    if (T == 0) return ORACLE_OK;
    if (!x || !wg || !wu || !wd || !out) return ORACLE_BAD_ARG;
    oracle_dims d;
    memset(&d, 0, sizeof d);
    d.hidden = H;  /* the fields expert_one reads */
    d.h_is_bf16 = h_is_bf16;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        double *hbuf = (double *)malloc(sizeof(double) * (size_t)I);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        if (!hbuf || !y) {
#pragma omp atomic write
            bad = 1;
        } else {
            expert_one(&d, I, x + (size_t)t * H, wg, wu, wd, hbuf, y);
            for (int n = 0; n < H; ++n) out[(size_t)t * H + n] = (float)y[n];
        }
        free(hbuf);
        free(y);
    }
    return bad ? ORACLE_BAD_ARG : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm between stacked layers (a workload choice, not from the pages):
 * x_next = bf16( y / sqrt(mean(y^2) + eps) ), unit gain, mean over H. */
int oracle_rmsnorm(int T, int H, const float *in, double eps, float *out)
{
    if (T < 0 || H <= 0 || (T > 0 && (!in || !out))) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int h = 0; h < H; ++h) ss += (double)in[(size_t)t * H + h] * (double)in[(size_t)t * H + h];
        double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int h = 0; h < H; ++h) out[(size_t)t * H + h] = (float)round_bf16((double)in[(size_t)t * H + h] * r);
    }
    return ORACLE_OK;
}

/* Round an array of doubles to bf16 values (exposed so the tests can check the
 * oracle's rounding against the format's definition on chosen values). */
void oracle_round_bf16(const double *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Block-scaled 4-bit expert weights.  The pages' low-bit builds store weights
 * in 4 bits ("Recursive launches Flint: open-weight coding model with 39.8
 * billion parameters for local execution", section "What Flint is, and how it
 * is built": 4-bit weights take roughly 23 GB;
 * Kalaris analysis: an NVFP4 build on NVIDIA hardware) without defining a
 * format for these kernels, so the format here is a definition: OCP
 * Microscaling MXFP4.
 *   element  FP4 E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
 *            exponent field 0 is subnormal (0.m), so the magnitudes are
 *            0, 0.5, 1, 1.5, 2, 3, 4, 6
 *   block    32 consecutive elements of a row (along the reduction dimension)
 *            share one scale
 *   scale    E8M0: byte s means 2^(s - 127) for s = 0..254; 255 is NaN
 *   packing  two elements per byte, the lower-indexed one in the low nibble
 * A weight is element x scale, exact in float32 for every code and scale, so
 * dequantisation returns float32 arrays that the layer functions above take
 * unchanged. */
static double e2m1_value(unsigned code)
{
    const unsigned e = (code >> 1) & 3u, m = code & 1u;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

static double e8m0_value(unsigned s) { return s == 255u ? NAN : ldexp(1.0, (int)s - 127); }

/* codes [rows][cols/2], scales [rows][cols/32] -> out [rows][cols] (cols % 32 == 0). */
int oracle_mx4_dequant(int64_t rows, int cols, const uint8_t *codes, const uint8_t *scales, float *out)
{
    if (rows < 0 || cols <= 0 || cols % 32 != 0 || (rows > 0 && (!codes || !scales || !out))) return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c) {
            const unsigned byte = codes[r * (cols / 2) + c / 2];
            const unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
            const unsigned sc = scales[r * (cols / 32) + c / 32];
            out[r * cols + c] = (float)(e2m1_value(code) * e8m0_value(sc));
        }
    return ORACLE_OK;
}

/* The library's storage order for these arrays (a definition, like the format):
 * a tile is 16 consecutive rows x one 32-element block; the tiles of a matrix
 * run along the columns, then down the rows; a tile holds its 16 rows' 16 code
 * bytes, row after row (256 bytes), and its 16 scale bytes, row after row.
 * Back to row-major, element by element of the definition:
 *   codes_t[rb][kb][r][j] -> codes[rb*16 + r][kb*16 + j]
 *   scales_t[rb][kb][r]   -> scales[rb*16 + r][kb]
 * rows % 16 == 0, cols % 32 == 0; stacked matrices ([E][rows][cols]) are one
 * matrix of E*rows rows, as their tile rows follow each other. */
int oracle_mx4_untile(int64_t rows, int cols, const uint8_t *codes_t, const uint8_t *scales_t, uint8_t *codes,
                      uint8_t *scales)
{
    if (rows < 0 || rows % 16 != 0 || cols <= 0 || cols % 32 != 0 ||
        (rows > 0 && (!codes_t || !scales_t || !codes || !scales)))
        return ORACLE_BAD_ARG;
    const int64_t nkb = cols / 32;
    for (int64_t rb = 0; rb < rows / 16; ++rb)
        for (int64_t kb = 0; kb < nkb; ++kb)
            for (int r = 0; r < 16; ++r) {
                const int64_t tile = rb * nkb + kb;
                for (int j = 0; j < 16; ++j)
                    codes[(rb * 16 + r) * (cols / 2) + kb * 16 + j] = codes_t[(tile * 16 + r) * 16 + j];
                scales[(rb * 16 + r) * nkb + kb] = scales_t[tile * 16 + r];
            }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Parameter counts of one MoE layer from its shape, gated three-matrix experts.
 * Source: serving-kit review, "The architecture, from the config" -- the page's
 * own hand count (routed experts about 37.8B over 47 layers; six experts plus
 * the shared expert about 1.2B per token).
 *   out[0] = router parameters            E*H
 *   out[1] = routed expert parameters     E * 3*H*I
 *   out[2] = one routed expert            3*H*I
 *   out[3] = shared expert                3*H*Is
 *   out[4] = active per token             K*3*H*I + 3*H*Is  (experts only) */
void oracle_param_counts(const oracle_dims *d, int64_t *out)
{
    const int64_t H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter;
    out[0] = E * H;
    out[1] = E * 3 * H * I;
    out[2] = 3 * H * I;
    out[3] = 3 * H * Is;
    out[4] = K * 3 * H * I + 3 * H * Is;
}

/* Threads the OpenMP loops over tokens use (1 without OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads of the loops over tokens (n >= 1; ignored
 * without OpenMP).  Used to time the oracle on one core and on all of them. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
