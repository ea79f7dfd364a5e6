/*
 * oracle.c -- plain, slow, float64 CPU definition of the sigmoid
 * group-limited MoE gate and of its expert-major dispatch.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the HIP path is
 * compared against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or
 * helper with the HIP library and includes nothing from it.
 *
 * Every step is written in the order the pages give it, with no blocking,
 * fusion or reordering:
 *
 *   gate   (DeepSeek-V3.2-Exp · Normalize weights, "Code": Gate forward;
 *           Kimi K2 · Normalize weights, "Code": gate forward;
 *           AI Engineer Exhaustive · DeepSeek-V3 MoE Router, "How it works")
 *     1. logits  L[t,e] = u_t . e_i        (x cast to float, no linear bias)
 *     2. affinity s = Sigmoid(L)           (eq. for s_{i,t})
 *     3. choice score v = s + b            (load-balance bias paragraph)
 *     4. group score = sum of the two largest v in the group
 *     5. keep the topk_group best groups, all other experts masked to -inf
 *     6. token top-K over the masked v
 *     7. gather the UNBIASED s at the winners
 *     8. renormalise over the K winners, multiply by route_scale
 *        (eq. for g'/g; Normalize-weights equation G_i)
 *
 *   options (DeepSeek-V3.2-Exp · Normalize weights, "Code"; Kimi K2 ·
 *   Normalize weights, "Code"):
 *     - score function softmax over the E logits instead of sigmoid;
 *     - no bias: choice score = affinity, group score = group maximum;
 *     - renormalisation: by default only for sigmoid (DeepSeek-V3.2-Exp),
 *       or forced on / off (Kimi K2 gates it on a config flag);
 *     - dropped groups filled with 0.0 instead of -inf, and an epsilon added
 *       to the renormalisation denominator (both as the Kimi K2 gate does).
 *
 *   dispatch (Kimi K2 · Add shared output, "Code": moe_infer, first lines)
 *     per-expert token counts, expert-major argsort of the flat (token, slot)
 *     pairs, and the row gather x[perm // K].
 *
 *   combine (Kimi K2 · Add shared output, "Code": moe_infer, last lines)
 *     un-permute the expert outputs and sum each token's K rows weighted by
 *     its gate weights: y[t] = sum_k w[t,k] * out[dest[t*K + k]].
 *
 * Readings taken where the pages leave a choice open:
 *   - arithmetic is float64 throughout (the pages use float32);
 *   - masked experts get -inf (DeepSeek-V3.2-Exp page and the study note;
 *     the Kimi K2 page fills 0.0);
 *   - every top-k breaks ties towards the LOWER index (experts and groups);
 *   - order 0 emits a token's K winners in ascending expert id, order 1 in
 *     selection order (v descending, index ascending);
 *   - the renormalisation has no epsilon in the denominator;
 *   - the dispatch permutation is stable: pairs of one expert keep ascending
 *     flat pair id p = t*K + k.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* bfloat16 bit pattern -> double.  A bfloat16 is the top half of a float32,
 * so the conversion is exact. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Validate a gate configuration: E experts in G equal groups of S = E/G,
 * keep KG groups, select K experts among the KG*S candidates. */
static int check_cfg(int64_t E, int G, int KG, int K)
{
    if (E <= 0 || G <= 0 || KG <= 0 || K <= 0) return ORACLE_EINVAL;
    if (E % G != 0) return ORACLE_EINVAL;
    if (KG > G) return ORACLE_EINVAL;
    if (G > 1 && E / G < 2) return ORACLE_EINVAL; /* top-2 of a group needs 2 members */
    if ((int64_t)K > (int64_t)KG * (E / G)) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* Step 1.  L[t,e] = sum_j x[t,j] * W[e,j] with W laid out [E, d] (expert
 * rows, as F.linear's weight).  Products of a bfloat16 and a float32 are
 * exact in double; only the sum rounds. */
static void logits_row(const uint16_t *x_row, const float *W, int64_t d,
                       int64_t E, double *L)
{
    for (int64_t e = 0; e < E; ++e) {
        const float *w = W + e * d;
        double acc = 0.0;
        for (int64_t j = 0; j < d; ++j)
            acc += bf16_to_double(x_row[j]) * (double)w[j];
        L[e] = acc;
    }
}

void oracle_logits(const uint16_t *x, const float *W, int64_t T, int64_t d,
                   int64_t E, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        logits_row(x + t * d, W, d, E, logits + t * E);
}

/* True when (va, a) comes before (vb, b) in "value descending, index
 * ascending" order. */
static int precedes(double va, int64_t a, double vb, int64_t b)
{
    if (va > vb) return 1;
    if (va < vb) return 0;
    return a < b;
}

/* Options beyond the default DeepSeek-V3 / Kimi-K2 gate. */
typedef struct {
    int score_func;    /* 0 sigmoid, 1 softmax over the E logits           */
    int renorm;        /* 0 auto (sigmoid: yes, softmax: no), 1 yes, 2 no  */
    int mask_zero;     /* dropped groups: 0 -> -inf, 1 -> 0.0              */
    double denom_eps;  /* added to the renormalisation denominator         */
} gate_opts;

/* Steps 2-4 for one token, from its E logits: affinities s, choice scores
 * v and (when G > 1) group scores gs.
 *   bias: [E] or NULL (no bias: choice score = affinity, group score =
 *         group maximum) */
static void token_scores(const double *L, const float *bias, int64_t E, int G,
                         const gate_opts *opt, double *s, double *v, double *gs)
{
    const int64_t S = E / G;

    /* Step 2: affinities. */
    if (opt->score_func == 0) {
        /* s = 1 / (1 + exp(-L)) */
        for (int64_t e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + exp(-L[e]));
    } else {
        /* s = exp(L) / sum exp(L), shifted by the maximum for range */
        double mx = -INFINITY, sum = 0.0;
        for (int64_t e = 0; e < E; ++e) mx = L[e] > mx ? L[e] : mx;
        for (int64_t e = 0; e < E; ++e) sum += exp(L[e] - mx);
        for (int64_t e = 0; e < E; ++e) s[e] = exp(L[e] - mx) / sum;
    }

    /* Step 3: the bias shifts the choice score only. */
    for (int64_t e = 0; e < E; ++e) v[e] = s[e] + (bias ? (double)bias[e] : 0.0);

    /* Step 4: group scores. */
    if (G > 1) {
        for (int g = 0; g < G; ++g) {
            /* two largest values of the group, counting multiplicity */
            double top1 = -INFINITY, top2 = -INFINITY;
            for (int64_t e = g * S; e < (g + 1) * S; ++e) {
                if (v[e] > top1) {
                    top2 = top1;
                    top1 = v[e];
                } else if (v[e] > top2) {
                    top2 = v[e];
                }
            }
            if (bias)
                gs[g] = top1 + top2;
            else
                gs[g] = top1;   /* no bias: the group maximum */
        }
    }
}

/* Steps 2-8 for one token, from its E logits.
 *   bias: [E] or NULL (no bias: choice score = affinity, group score =
 *         group maximum)
 *   scratch: s, v, mv of E doubles; keep, gs of G; chosen of E; sel of K
 *   out_w[K], out_i[K]: weights and expert ids
 *   margin[2]: {K-th minus (K+1)-th masked choice score,
 *               KG-th minus (KG+1)-th group score}; +inf when undefined. */
static void select_token(const double *L, const float *bias, int64_t E, int G,
                         int KG, int K, double route_scale, int order,
                         const gate_opts *opt, double *s, double *v,
                         double *mv, int *keep, double *gs, int *chosen,
                         int64_t *sel, double *out_w, int32_t *out_i,
                         double *margin)
{
    const int64_t S = E / G;

    /* Steps 2-4: affinities, choice scores, group scores. */
    token_scores(L, bias, E, G, opt, s, v, gs);

    /* Step 5: group keep mask. */
    for (int g = 0; g < G; ++g) keep[g] = 1;
    margin[1] = INFINITY;
    if (G > 1) {
        /* a group is kept when fewer than KG groups precede it */
        for (int g = 0; g < G; ++g) {
            int ahead = 0;
            for (int h = 0; h < G; ++h)
                if (h != g && precedes(gs[h], h, gs[g], g)) ++ahead;
            keep[g] = ahead < KG;
        }
        if (KG < G) {
            /* KG-th and (KG+1)-th largest group scores */
            double kth = -INFINITY, next = -INFINITY;
            for (int g = 0; g < G; ++g) {
                int ahead = 0;
                for (int h = 0; h < G; ++h)
                    if (h != g && precedes(gs[h], h, gs[g], g)) ++ahead;
                if (ahead == KG - 1) kth = gs[g];
                if (ahead == KG) next = gs[g];
            }
            margin[1] = kth - next;
        }
    }

    /* Step 5: experts of dropped groups take the fill value. */
    const double fill = opt->mask_zero ? 0.0 : -INFINITY;
    for (int64_t e = 0; e < E; ++e) mv[e] = keep[e / S] ? v[e] : fill;

    /* Step 6: repeatedly take the best remaining expert of the masked
     * scores.  With the -inf fill, dropped experts are never taken because
     * K <= KG*S. */
    for (int64_t e = 0; e < E; ++e) chosen[e] = 0;
    for (int k = 0; k < K; ++k) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (chosen[e]) continue;
            if (best < 0 || precedes(mv[e], e, mv[best], best)) best = e;
        }
        chosen[best] = 1;
        sel[k] = best;
    }
    /* margin between the K-th winner and the best loser */
    {
        double best_loser = -INFINITY;
        int any = 0;
        for (int64_t e = 0; e < E; ++e) {
            if (chosen[e] || mv[e] == -INFINITY) continue;
            if (!any || mv[e] > best_loser) best_loser = mv[e];
            any = 1;
        }
        margin[0] = any ? mv[sel[K - 1]] - best_loser : INFINITY;
    }

    /* canonical order: ascending expert id */
    if (order == 0) {
        for (int a = 1; a < K; ++a) {
            int64_t key = sel[a];
            int b = a - 1;
            while (b >= 0 && sel[b] > key) {
                sel[b + 1] = sel[b];
                --b;
            }
            sel[b + 1] = key;
        }
    }

    /* Steps 7-8: gather unbiased s, renormalise, scale. */
    const int renorm = opt->renorm == 0 ? opt->score_func == 0 : opt->renorm == 1;
    double denom = 0.0;
    for (int k = 0; k < K; ++k) denom += s[sel[k]];
    denom += opt->denom_eps;
    for (int k = 0; k < K; ++k) {
        out_i[k] = (int32_t)sel[k];
        if (renorm)
            out_w[k] = s[sel[k]] / denom * route_scale;
        else
            out_w[k] = s[sel[k]] * route_scale;
    }
}

static int check_opts(int score_func, int renorm, int mask_zero)
{
    if (score_func != 0 && score_func != 1) return ORACLE_EINVAL;
    if (renorm < 0 || renorm > 2) return ORACLE_EINVAL;
    if (mask_zero != 0 && mask_zero != 1) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* Gate from precomputed float64 logits [T, E]; bias may be NULL.
 *   margins may be NULL; otherwise [T, 2]. */
int oracle_select(const double *logits, const float *bias, int64_t T,
                  int64_t E, int G, int KG, int K, double route_scale,
                  int order, int score_func, int renorm, int mask_zero,
                  double denom_eps, double *weights, int32_t *indices,
                  double *margins)
{
    if (check_cfg(E, G, KG, K) != ORACLE_OK) return ORACLE_EINVAL;
    if (order != 0 && order != 1) return ORACLE_EINVAL;
    if (check_opts(score_func, renorm, mask_zero) != ORACLE_OK) return ORACLE_EINVAL;
    const gate_opts opt = {score_func, renorm, mask_zero, denom_eps};
    int failed = 0;
#pragma omp parallel
    {
        double *s = malloc(sizeof(double) * E);
        double *v = malloc(sizeof(double) * E);
        double *mv = malloc(sizeof(double) * E);
        double *gs = malloc(sizeof(double) * G);
        int *keep = malloc(sizeof(int) * G);
        int *chosen = malloc(sizeof(int) * E);
        int64_t *sel = malloc(sizeof(int64_t) * K);
        double mdummy[2];
        if (!s || !v || !mv || !gs || !keep || !chosen || !sel) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t)
                select_token(logits + t * E, bias, E, G, KG, K, route_scale,
                             order, &opt, s, v, mv, keep, gs, chosen, sel,
                             weights + t * K, indices + t * K,
                             margins ? margins + 2 * t : mdummy);
        }
        free(s); free(v); free(mv); free(gs); free(keep); free(chosen); free(sel);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/* Steps 2-4 from precomputed float64 logits [T, E]: affinities s [T, E],
 * choice scores v [T, E] and group scores gs [T, G] (gs is not written when
 * G == 1).  bias may be NULL; score_func as in oracle_select. */
int oracle_scores(const double *logits, const float *bias, int64_t T, int64_t E,
                  int G, int score_func, double *s, double *v, double *gs)
{
    if (E <= 0 || G <= 0 || E % G != 0) return ORACLE_EINVAL;
    if (G > 1 && E / G < 2) return ORACLE_EINVAL;
    if (score_func != 0 && score_func != 1) return ORACLE_EINVAL;
    const gate_opts opt = {score_func, 0, 0, 0.0};
    int failed = 0;
#pragma omp parallel
    {
        double *gdummy = malloc(sizeof(double) * G);
        if (!gdummy) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t)
                token_scores(logits + t * E, bias, E, G, &opt, s + t * E, v + t * E,
                             G > 1 ? gs + t * G : gdummy);
        }
        free(gdummy);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/* Whole gate from x (bfloat16 bits, [T, d]), W (float32, [E, d]) and bias
 * (float32, [E], or NULL).  Logits are computed token by token and never
 * stored. */
int oracle_gate(const uint16_t *x, const float *W, const float *bias,
                int64_t T, int64_t d, int64_t E, int G, int KG, int K,
                double route_scale, int order, int score_func, int renorm,
                int mask_zero, double denom_eps, double *weights,
                int32_t *indices, double *margins)
{
    if (check_cfg(E, G, KG, K) != ORACLE_OK || d <= 0) return ORACLE_EINVAL;
    if (order != 0 && order != 1) return ORACLE_EINVAL;
    if (check_opts(score_func, renorm, mask_zero) != ORACLE_OK) return ORACLE_EINVAL;
    const gate_opts opt = {score_func, renorm, mask_zero, denom_eps};
    int failed = 0;
#pragma omp parallel
    {
        double *L = malloc(sizeof(double) * E);
        double *s = malloc(sizeof(double) * E);
        double *v = malloc(sizeof(double) * E);
        double *mv = malloc(sizeof(double) * E);
        double *gs = malloc(sizeof(double) * G);
        int *keep = malloc(sizeof(int) * G);
        int *chosen = malloc(sizeof(int) * E);
        int64_t *sel = malloc(sizeof(int64_t) * K);
        double mdummy[2];
        if (!L || !s || !v || !mv || !gs || !keep || !chosen || !sel) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                logits_row(x + t * d, W, d, E, L);
                select_token(L, bias, E, G, KG, K, route_scale, order, &opt,
                             s, v, mv, keep, gs, chosen, sel, weights + t * K,
                             indices + t * K,
                             margins ? margins + 2 * t : mdummy);
            }
        }
        free(L); free(s); free(v); free(mv); free(gs); free(keep); free(chosen);
        free(sel);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/* Dispatch metadata from indices [T, K] (flat pair p = t*K + k):
 *   counts[E]      tokens routed to each expert
 *   offsets[E+1]   exclusive prefix sum of counts
 *   perm[T*K]      perm[pos] = p, expert-major, ascending p within an expert
 * This is a counting sort that walks the pairs in ascending p. */
int oracle_dispatch(const int32_t *indices, int64_t T, int K, int64_t E,
                    int32_t *counts, int32_t *offsets, int32_t *perm)
{
    const int64_t n = T * (int64_t)K;
    if (T < 0 || K <= 0 || E <= 0) return ORACLE_EINVAL;
    for (int64_t p = 0; p < n; ++p)
        if (indices[p] < 0 || indices[p] >= E) return ORACLE_EINVAL;

    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < n; ++p) counts[indices[p]] += 1;

    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    int32_t *fill = malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return ORACLE_EINVAL;
    for (int64_t e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t p = 0; p < n; ++p) {
        int32_t e = indices[p];
        perm[fill[e]] = (int32_t)p;
        fill[e] += 1;
    }
    free(fill);
    return ORACLE_OK;
}

/* Row gather: out[pos, :] = x[perm[pos] / K, :] for pos < n (bfloat16 bits,
 * rows of d elements). */
int oracle_gather_rows(const uint16_t *x, int64_t T, int64_t d, int K,
                       const int32_t *perm, int64_t n, uint16_t *out)
{
    for (int64_t pos = 0; pos < n; ++pos) {
        int64_t p = perm[pos];
        if (p < 0 || p / K >= T) return ORACLE_EINVAL;
        memcpy(out + pos * d, x + (p / K) * d, sizeof(uint16_t) * (size_t)d);
    }
    return ORACLE_OK;
}

/* Combine: y[t, :] = sum_k w[t, k] * out[dest[t*K + k], :], where out is
 * the expert output in dispatch (expert-major) order, bfloat16 bits
 * [n_pos, d], and dest[p] is the position of pair p = t*K + k.  The sum is
 * float64 in ascending k; y64 receives it, and y16 (if not NULL) receives
 * it rounded to float32 and then to bfloat16 (round to nearest even), the
 * two roundings of a float32 sum cast back to the activation type. */
int oracle_combine(const uint16_t *out, int64_t n_pos, const double *w,
                   const int32_t *dest, int64_t T, int K, int64_t d,
                   double *y64, uint16_t *y16)
{
    for (int64_t p = 0; p < T * (int64_t)K; ++p)
        if (dest[p] < 0 || dest[p] >= n_pos) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                const int64_t pos = dest[t * K + k];
                acc += w[t * K + k] * bf16_to_double(out[pos * d + j]);
            }
            y64[t * d + j] = acc;
            if (y16) {
                float f = (float)acc;
                uint32_t u;
                memcpy(&u, &f, sizeof u);
                u += 0x7fffu + ((u >> 16) & 1u);   /* round to nearest even */
                y16[t * d + j] = (uint16_t)(u >> 16);
            }
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------
 * Expert-parallel metadata on one GPU (Kimi K2 · Add shared output,
 * "Code": moe_infer, the ep_size > 1 branch).  Experts are split into
 * ep_size ranks of experts_per_rank = E / ep_size consecutive experts.
 * ------------------------------------------------------------------- */

/* Rows each rank receives from this one: the per-rank sums of
 * tokens_per_expert (the pages' tokens_per_ep_rank / input_split_sizes),
 * and their exclusive prefix. */
int oracle_ep_send_splits(const int32_t *tokens_per_expert, int64_t E, int ep_size,
                          int32_t *send_counts, int32_t *send_offsets)
{
    if (ep_size <= 0 || E % ep_size != 0) return ORACLE_EINVAL;
    const int64_t per = E / ep_size;
    send_offsets[0] = 0;
    for (int r = 0; r < ep_size; ++r) {
        int32_t c = 0;
        for (int64_t j = 0; j < per; ++j) c += tokens_per_expert[r * per + j];
        send_counts[r] = c;
        send_offsets[r + 1] = send_offsets[r] + c;
    }
    return ORACLE_OK;
}

/* Receive-side regroup.  counts[r * per + j] rows arrive from source rank r
 * for local expert j, rank after rank and, within a rank, in local-expert
 * order.  Each received row is labelled with its local expert id; the rows
 * are then put in label order (the pages' argsort of gatherd_idxs), stably,
 * so rows of one expert keep their arrival order.
 *   local_counts[j] = sum_r counts[r, j]   (tokens_per_expert_post_gather)
 *   regroup[q] = index of the received row that goes to position q. */
int oracle_ep_regroup(const int32_t *counts, int ep_size, int64_t per,
                      int32_t *local_counts, int32_t *regroup)
{
    if (ep_size <= 0 || per <= 0) return ORACLE_EINVAL;
    int64_t n = 0;
    for (int64_t i = 0; i < ep_size * per; ++i) {
        if (counts[i] < 0) return ORACLE_EINVAL;
        n += counts[i];
    }
    int32_t *label = malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    if (!label) return ORACLE_EINVAL;
    int64_t s = 0;
    for (int r = 0; r < ep_size; ++r)
        for (int64_t j = 0; j < per; ++j)
            for (int32_t c = 0; c < counts[r * per + j]; ++c) label[s++] = (int32_t)j;
    /* stable counting sort of the labels */
    for (int64_t j = 0; j < per; ++j) local_counts[j] = 0;
    for (int64_t i = 0; i < n; ++i) local_counts[label[i]] += 1;
    int32_t *fill = malloc(sizeof(int32_t) * (size_t)per);
    if (!fill) { free(label); return ORACLE_EINVAL; }
    int32_t run = 0;
    for (int64_t j = 0; j < per; ++j) { fill[j] = run; run += local_counts[j]; }
    for (int64_t i = 0; i < n; ++i) regroup[fill[label[i]]++] = (int32_t)i;
    free(fill);
    free(label);
    return ORACLE_OK;
}

/* De-duplicated send list: a token whose top-K experts sit on one rank
 * several times is sent to that rank once.  For rank r = e / per:
 *   rank_counts[r]       distinct tokens sent to rank r
 *   rank_offsets[r]      exclusive prefix of rank_counts
 *   send_tokens[pos]     token ids, rank-major, ascending token inside a rank
 *   pair_slot[t*K + k]   position in send_tokens of (t, rank of its k-th expert)
 * Walks the tokens in ascending order and, per token, its K slots in order. */
int oracle_ep_dedup(const int32_t *indices, int64_t T, int K, int64_t E, int ep_size,
                    int32_t *rank_counts, int32_t *rank_offsets, int32_t *send_tokens,
                    int32_t *pair_slot)
{
    if (ep_size <= 0 || E % ep_size != 0 || K <= 0) return ORACLE_EINVAL;
    const int64_t per = E / ep_size;
    for (int64_t p = 0; p < T * K; ++p)
        if (indices[p] < 0 || indices[p] >= E) return ORACLE_EINVAL;
    for (int r = 0; r < ep_size; ++r) rank_counts[r] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < ep_size; ++r) {
            int hit = 0;
            for (int k = 0; k < K; ++k) hit |= indices[t * K + k] / per == r;
            rank_counts[r] += hit;
        }
    rank_offsets[0] = 0;
    for (int r = 0; r < ep_size; ++r) rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];
    int32_t *fill = malloc(sizeof(int32_t) * (size_t)ep_size);
    if (!fill) return ORACLE_EINVAL;
    for (int r = 0; r < ep_size; ++r) fill[r] = rank_offsets[r];
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            const int r = (int)(indices[t * K + k] / per);
            int first = k;   /* first slot of this token on rank r */
            for (int k2 = 0; k2 < k; ++k2)
                if (indices[t * K + k2] / per == r) { first = k2; break; }
            if (first == k) {
                send_tokens[fill[r]] = (int32_t)t;
                pair_slot[t * K + k] = fill[r];
                fill[r] += 1;
            } else {
                pair_slot[t * K + k] = pair_slot[t * K + first];
            }
        }
    }
    free(fill);
    return ORACLE_OK;
}
