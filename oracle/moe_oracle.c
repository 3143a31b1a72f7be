/*
 * CPU oracle of the MoE FFN layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  The HIP library never includes, links or calls it, and it
 * shares no code with the HIP sources.
 *
 * It computes the plain definitions in fp64, one token at a time, with no
 * blocking, fusion or reordering:
 *
 *  - routing: each token goes to the k best of E experts plus an always-on
 *    shared expert (page "Perplexity's Lily Beats MLX-LM by 1.35x Running
 *    Qwen3.6 on Apple Silicon", section "What Lily actually does"); the
 *    expert grouping is the counting sort that a histogram, a prefix scan, a
 *    scatter and a block-map build produce (same page, section "Prefill
 *    optimizations", second bullet);
 *  - weights are groupwise affine 4-bit codes, w = s*q + b per group of G
 *    consecutive input elements (same page and section, first paragraph;
 *    page "Perplexity Open Sources Lily: Rust & Metal Engine for Qwen3.6",
 *    paragraph on the 70 GB -> 19.4 GB quantisation);
 *  - every expert is a SwiGLU MLP, o = W_down (silu(W_gate x) * (W_up x)),
 *    and the layer output is sum_j w_j o_j + o_shared;
 *  - the router scores each token against every expert: logits = x W_r
 *    (+ a per-expert bias), W_r fp32 [d][E] (the step before the routing on
 *    the same page, section "What Lily actually does": each token's router
 *    picks its experts);
 *  - a second workload, decode attention of one token over grouped KV heads
 *    (eight query heads share one KV head: same page, section "Decode
 *    optimizations"), as scaled dot-product attention (oracle_gqa_decode).
 *
 * Readings of what the pages leave open (each is pinned by a CPU test):
 *  - top-k order: larger logit first, ties to the lower expert id, -0 == +0;
 *  - routing weights: softmax over the k selected logits (they sum to 1);
 *  - shared expert: same 4-bit format as routed experts, weight 1; or, when
 *    a gate vector g (bf16 [d]) is given, weight sigmoid(x . g) per token
 *    (the pages name the always-on shared expert and nothing more; the
 *    gated form is the optional variant of the library);
 *  - the scatter is stable: inside one expert, assignments a = t*k + j keep
 *    ascending order;
 *  - block map: for each expert in id order, tiles of tile_m consecutive
 *    sorted rows, the last one short;
 *  - code layout: W[n][i] has code byte q[n][i/2], element 2m in the low
 *    nibble, 2m+1 in the high nibble; scale/bias index [n][i/G].
 *
 * Precision: the exact weight s*q + b is formed in fp64 (s*q has at most 12
 * significant bits, so the sum is exact whenever the two terms are within
 * 2^40 of each other, which holds for every workload here).  The bf16 form
 * that a matrix-core kernel multiplies is defined as bf16_rne(fp32_rne(w));
 * the FFN itself uses the exact w and keeps h in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    const uint8_t *q;  /* [rows][cols/2] codes */
    const uint16_t *s; /* [rows][cols/G] bf16 scales */
    const uint16_t *b; /* [rows][cols/G] bf16 biases */
} omat;

typedef struct {
    omat gate, up, down;    /* routed, expert-major: [E][F][d], [E][F][d], [E][d][F] */
    omat sgate, sup, sdown; /* shared: [Fs][d], [Fs][d], [d][Fs] */
} oweights;

static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* 4-bit code of element (n, i) of a [rows][cols] matrix */
static int code_at(const omat *m, int cols, int n, int i)
{
    uint8_t byte = m->q[(size_t)n * (size_t)(cols / 2) + (size_t)(i / 2)];
    return (i & 1) ? (byte >> 4) : (byte & 15);
}

/* exact dequantised value w = s*q + b of element (n, i) */
static double weight_at(const omat *m, int cols, int G, int n, int i)
{
    size_t gi = (size_t)n * (size_t)(cols / G) + (size_t)(i / G);
    return bf16_value(m->s[gi]) * (double)code_at(m, cols, n, i) + bf16_value(m->b[gi]);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- dequant */

void oracle_dequant_exact(const uint8_t *q, const uint16_t *s, const uint16_t *b,
                          int rows, int cols, int G, double *out)
{
    omat m = {q, s, b};
    for (int n = 0; n < rows; ++n)
        for (int i = 0; i < cols; ++i)
            out[(size_t)n * cols + i] = weight_at(&m, cols, G, n, i);
}

void oracle_dequant_bf16(const uint8_t *q, const uint16_t *s, const uint16_t *b,
                         int rows, int cols, int G, uint16_t *out)
{
    omat m = {q, s, b};
    for (int n = 0; n < rows; ++n)
        for (int i = 0; i < cols; ++i)
            out[(size_t)n * cols + i] = bf16_rne((float)weight_at(&m, cols, G, n, i));
}

/* ---------------------------------------------------------------- routing */

/* k rounds of "best remaining expert": larger logit wins, equal logits go to
 * the lower id (ids are scanned in ascending order and only a strictly larger
 * logit replaces the current best).  C's '>' treats -0 and +0 as equal. */
void oracle_topk(int T, int E, int k, const float *logits, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *L = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || L[e] > L[best])) best = e;
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        /* softmax over the selected logits; the first one is the largest */
        double lmax = (double)L[ids[(size_t)t * k]], sum = 0.0;
        for (int j = 0; j < k; ++j) {
            double e = exp((double)L[ids[(size_t)t * k + j]] - lmax);
            w[(size_t)t * k + j] = e;
            sum += e;
        }
        for (int j = 0; j < k; ++j) w[(size_t)t * k + j] /= sum;
    }
    free(taken);
}

/* histogram -> exclusive prefix sum -> stable scatter, as a counting sort of
 * the T*k assignments a = t*k + j by expert id. */
void oracle_counting_sort(int T, int E, int k, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv_perm)
{
    int64_t A = (int64_t)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < A; ++a) counts[ids[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t p = 0;
    for (int e = 0; e < E; ++e)
        for (int64_t a = 0; a < A; ++a)
            if (ids[a] == e) perm[p++] = (int32_t)a;
    for (int64_t q = 0; q < A; ++q) inv_perm[perm[q]] = (int32_t)q;
}

/* tiles (expert, first sorted row, rows) covering every expert's rows in
 * chunks of tile_m; returns the tile count, or -1 if it exceeds max_tiles. */
int oracle_block_map(int E, const int32_t *counts, const int32_t *offsets, int tile_m,
                     int max_tiles, int32_t *tile_expert, int32_t *tile_row0, int32_t *tile_rows)
{
    int n = 0;
    for (int e = 0; e < E; ++e)
        for (int r0 = 0; r0 < counts[e]; r0 += tile_m) {
            if (n >= max_tiles) return -1;
            tile_expert[n] = e;
            tile_row0[n] = offsets[e] + r0;
            tile_rows[n] = (counts[e] - r0 < tile_m) ? counts[e] - r0 : tile_m;
            ++n;
        }
    return n;
}

/* ---------------------------------------------------------------- FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* one SwiGLU expert on one token: out[d] = W_down (silu(W_gate x) * W_up x).
 * gate/up are [Fw][d], down is [d][Fw]; h is scratch of Fw doubles. */
static void expert_ffn(const omat *gate, const omat *up, const omat *down, int d, int Fw, int G,
                       const double *x, double *h, double *out)
{
    for (int n = 0; n < Fw; ++n) {
        double g = 0.0, u = 0.0;
        for (int i = 0; i < d; ++i) {
            double wg = weight_at(gate, d, G, n, i), wu = weight_at(up, d, G, n, i);
            g += wg * x[i];
            u += wu * x[i];
        }
        h[n] = silu(g) * u;
    }
    for (int i = 0; i < d; ++i) {
        double o = 0.0;
        for (int n = 0; n < Fw; ++n) {
            double wd = weight_at(down, Fw, G, i, n);
            o += wd * h[n];
        }
        out[i] = o;
    }
}

static omat expert_slab(const omat *m, int e, int rows, int cols, int G)
{
    omat r;
    r.q = m->q + (size_t)e * rows * (cols / 2);
    r.s = m->s + (size_t)e * rows * (cols / G);
    r.b = m->b + (size_t)e * rows * (cols / G);
    return r;
}

/* Weight of the shared expert for token x: 1 without a gate vector, else
 * the logistic sigmoid of the dot product x . g (fp64). */
static double shared_weight(const double *x, const uint16_t *g, int d)
{
    if (!g) return 1.0;
    double z = 0.0;
    for (int i = 0; i < d; ++i) z += x[i] * bf16_value(g[i]);
    return 1.0 / (1.0 + exp(-z));
}

/* y[ti][:] for the tokens tokens[0..ntok) (all T tokens if tokens == NULL):
 * y = sum_j w[t][j] * FFN_{ids[t][j]}(x_t) + gamma_t * FFN_shared(x_t), in
 * fp64, gamma_t = shared_weight(x_t, shared_gate). */
void oracle_ffn(int T, int d, int E, int k, int F, int Fs, int G, const uint16_t *x,
                const oweights *W, const uint16_t *shared_gate, const int32_t *ids, const double *w,
                const int32_t *tokens, int ntok, double *y)
{
    (void)E;
    int n_out = tokens ? ntok : T;
    int Fmax = F > Fs ? F : Fs;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ti = 0; ti < n_out; ++ti) {
        int t = tokens ? tokens[ti] : ti;
        double *xt = (double *)malloc(sizeof(double) * (size_t)d);
        double *h = (double *)malloc(sizeof(double) * (size_t)Fmax);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double *yt = y + (size_t)ti * d;
        for (int i = 0; i < d; ++i) xt[i] = bf16_value(x[(size_t)t * d + i]);
        for (int i = 0; i < d; ++i) yt[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            omat g = expert_slab(&W->gate, e, F, d, G);
            omat u = expert_slab(&W->up, e, F, d, G);
            omat dn = expert_slab(&W->down, e, d, F, G);
            expert_ffn(&g, &u, &dn, d, F, G, xt, h, o);
            for (int i = 0; i < d; ++i) yt[i] += w[(size_t)t * k + j] * o[i];
        }
        expert_ffn(&W->sgate, &W->sup, &W->sdown, d, Fs, G, xt, h, o);
        const double gamma = shared_weight(xt, shared_gate, d);
        for (int i = 0; i < d; ++i) yt[i] += gamma * o[i];
        free(xt);
        free(h);
        free(o);
    }
}

/* Router logits: L[t][e] = sum_i x[t][i] W[i][e] (+ bias[e]), x bf16 [T][d],
 * W fp32 [d][E], bias fp32 [E] or NULL, fp64 sums in input order. */
void oracle_router_logits(int T, int d, int E, const uint16_t *x, const float *W, const float *bias,
                          double *L)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += bf16_value(x[(size_t)t * d + i]) * (double)W[(size_t)i * E + e];
            if (bias) acc += (double)bias[e];
            L[(size_t)t * E + e] = acc;
        }
}

/* Decode attention of one token over grouped KV heads (a second workload of
 * the pages: page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on
 * Apple Silicon", section "Decode optimizations": eight query heads share one
 * KV head; the model's full-attention layers: page "Perplexity Open Sources
 * Lily Inference Engine for Apple Silicon", opening paragraphs).  The pages do
 * not write the formula; this is scaled dot-product attention.  Query head h
 * reads KV head g = h / (Hq / Hkv):
 *   s_t = (q_h . k_{g,t}) / sqrt(D),  p_t = exp(s_t - max s) / sum_u exp(s_u - max s),
 *   o_h = sum_t p_t v_{g,t},
 * in fp64 from bf16 inputs: q [Hq][D], k and v [Hkv][L][D] (token rows),
 * out [Hq][D]. */
void oracle_gqa_decode(int Hq, int Hkv, int D, int L, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, double *out)
{
    const int G = Hq / Hkv;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; ++h) {
        const int g = h / G;
        double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double smax = -INFINITY;
        for (int t = 0; t < L; ++t) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i)
                acc += bf16_value(q[(size_t)h * D + i]) * bf16_value(k[((size_t)g * L + t) * D + i]);
            s[t] = acc / sqrt((double)D);
            if (s[t] > smax) smax = s[t];
        }
        double den = 0.0;
        for (int t = 0; t < L; ++t) {
            s[t] = exp(s[t] - smax);
            den += s[t];
        }
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int t = 0; t < L; ++t) acc += s[t] * bf16_value(v[((size_t)g * L + t) * D + i]);
            out[(size_t)h * D + i] = acc / den;
        }
        free(s);
    }
}
