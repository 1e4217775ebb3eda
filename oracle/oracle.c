/*
 * CPU oracle for the forward pass of one mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the
 * HIP path is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Everything is computed token by token in double precision from the exact
 * stored input values (bfloat16 and float32 widen exactly to double).  No
 * intermediate is rounded to a narrower type.  Loops are plain; the only
 * parallelism is a static split of independent tokens over threads.
 *
 * Sources (pages as titled):
 *  - "Expert Parallelism (MoE)", section "MoE Layer Structure": the router is a
 *    Linear d -> N_experts giving per-token expert ids, the top-K experts are
 *    activated, each expert is Linear(d->4d) -> GELU -> Linear(4d->d), and the
 *    output is the routing-weighted sum over the selected experts.
 *  - same page, section "Load Balancing: The Auxiliary Loss": L_aux, f_i, P_i
 *    and the balancing weight alpha.
 *  - same page, section "Top-K Routing and Capacity Factor": capacity and the
 *    dropping of tokens that would push an expert over it, with their routing
 *    weight zeroed.
 *  - "Expert Parallelism (EP)", section "Key math / How it works": route,
 *    dispatch to the expert's owner, expert GEMMs, combine back home.
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reasons in the design notes of the repository):
 *  - routing probabilities are the softmax over all E logits; the routing
 *    weight of a selected expert is that probability, not renormalised;
 *  - top-k orders experts by logit, descending, ties to the lower expert id;
 *  - f_i = (selections of expert i before any capacity cap) / T and
 *    P_i = mean over tokens of the softmax probability of expert i;
 *  - capacity C = floor(T * capacity_factor / E); an expert keeps the first C
 *    (token, slot) selections in token-index order; the rest are dropped;
 *  - GELU is the exact erf form;
 *  - a shared expert, when present, runs on every token with weight 1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_DT_F32 0
#define ORACLE_DT_BF16 1

/* Value i of an array stored as float32 or as bfloat16 bit patterns. */
static double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_DT_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/* ---------------------------------------------------------------------- */
/* threads                                                                 */
/* ---------------------------------------------------------------------- */

typedef void (*range_fn)(void *ctx, int64_t begin, int64_t end);

struct range_job {
    range_fn fn;
    void *ctx;
    int64_t begin, end;
};

static void *run_range(void *p)
{
    struct range_job *j = (struct range_job *)p;
    if (j->begin < j->end)
        j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

/* Split [0, n) into nthreads contiguous pieces and run fn on each. */
static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx)
{
    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > n)
        nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    struct range_job *jobs = (struct range_job *)calloc((size_t)nthreads, sizeof(struct range_job));
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].begin = n * i / nthreads;
        jobs[i].end = n * (i + 1) / nthreads;
        pthread_create(&th[i], NULL, run_range, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

/* ---------------------------------------------------------------------- */
/* Router: logits, softmax, top-k, routing weights                         */
/* ---------------------------------------------------------------------- */

struct route_ctx {
    const void *x;
    int x_dtype;
    const float *w_router, *b_router, *sel_bias;
    int d, E, k;
    double *logits, *probs, *topk_w;
    int32_t *topk_idx;
};

static void route_range(void *p, int64_t t0, int64_t t1)
{
    struct route_ctx *c = (struct route_ctx *)p;
    const int d = c->d, E = c->E, k = c->k;
    double *lg = (double *)malloc(sizeof(double) * (size_t)E);
    double *sc = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int64_t t = t0; t < t1; ++t) {
        /* Router Linear d -> E ("MoE Layer Structure"). */
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += elem(c->x, c->x_dtype, t * d + i) * (double)c->w_router[(int64_t)e * d + i];
            if (c->b_router)
                s += (double)c->b_router[e];
            lg[e] = s;
        }
        /* Softmax over all E experts. */
        double mx = lg[0];
        for (int e = 1; e < E; ++e)
            if (lg[e] > mx)
                mx = lg[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp(lg[e] - mx);
        double *pr = c->probs + t * E;
        for (int e = 0; e < E; ++e)
            pr[e] = exp(lg[e] - mx) / z;
        if (c->logits)
            memcpy(c->logits + t * E, lg, sizeof(double) * (size_t)E);
        /* Selection score: the logit, plus the per-expert selection-only
         * bias when one is given ("Expert Parallelism (EP)", load balancing:
         * DeepSeek-V3's bias adjustment instead of the auxiliary loss).  The
         * bias steers which experts are chosen; the weights below stay the
         * unbiased softmax probabilities. */
        for (int e = 0; e < E; ++e)
            sc[e] = c->sel_bias ? lg[e] + (double)c->sel_bias[e] : lg[e];
        /* Top-k: repeatedly take the largest remaining score; scanning ids
         * upward with a strict comparison keeps the lower id on a tie. */
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || sc[e] > sc[best])
                    best = e;
            }
            taken[best] = 1;
            c->topk_idx[t * k + j] = best;
            c->topk_w[t * k + j] = pr[best];
        }
    }
    free(lg);
    free(sc);
    free(taken);
}

/* Route T tokens.  x is [T, d] (float32 or bfloat16 bits per x_dtype),
 * w_router [E, d] float32, b_router [E] float32 or NULL, sel_bias [E] float32
 * or NULL (selection-only bias).  Outputs: logits [T, E] (may be NULL), probs
 * [T, E], topk_idx [T, k], topk_w [T, k].  Returns 0, or -1 on invalid sizes. */
int oracle_route(const void *x, int x_dtype, const float *w_router, const float *b_router,
                 const float *sel_bias, int64_t T, int d, int E, int k, double *logits, double *probs,
                 int32_t *topk_idx, double *topk_w, int nthreads)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E)
        return -1;
    struct route_ctx c = {x, x_dtype, w_router, b_router, sel_bias, d, E, k, logits, probs, topk_w, topk_idx};
    parallel_for(T, nthreads, route_range, &c);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Load statistics ("Load Balancing: The Auxiliary Loss")                   */
/* ---------------------------------------------------------------------- */

/* count[e]: selections of expert e over all (token, slot), before capacity.
 * f[e] = count[e] / T.  P[e] = mean over tokens of probs[t, e].
 * l_aux = alpha * sum_e f[e] * P[e]. */
int oracle_load_stats(const int32_t *topk_idx, const double *probs, int64_t T, int E, int k,
                      double alpha, int64_t *count, double *f, double *P, double *l_aux)
{
    if (T < 0 || E < 1 || k < 1)
        return -1;
    for (int e = 0; e < E; ++e) {
        count[e] = 0;
        P[e] = 0.0;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = topk_idx[t * k + j];
            if (e >= 0 && e < E)
                count[e] += 1;
        }
    for (int e = 0; e < E; ++e) {
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t)
            s += probs[t * E + e];
        P[e] = T > 0 ? s / (double)T : 0.0;
        f[e] = T > 0 ? (double)count[e] / (double)T : 0.0;
    }
    double acc = 0.0;
    for (int e = 0; e < E; ++e)
        acc += f[e] * P[e];
    *l_aux = alpha * acc;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Capacity, dropping and the expert-contiguous order                       */
/* ---------------------------------------------------------------------- */

/* Capacity C = floor(T * capacity_factor / E) ("Top-K Routing and Capacity
 * Factor"); capacity_factor <= 0 means no cap (C is reported as -1).
 *
 * Walk the selections in token order (t ascending, then slot j).  A selection
 * of an expert outside the local range [e0, e0 + E_loc) is remote (-2).  A
 * local selection is kept while its expert has seen fewer than C selections,
 * otherwise dropped (-1).  Kept selections are then laid out expert by expert
 * (experts ascending, tokens ascending inside an expert): seg_offsets is the
 * exclusive scan of kept_count, slot_row[t*k+j] the row of a kept selection,
 * and row_src[row] = t*k+j. */
int oracle_capacity(const int32_t *topk_idx, int64_t T, int E, int k, double capacity_factor,
                    int e0, int E_loc, int64_t *capacity, int32_t *slot_row, int32_t *row_src,
                    int32_t *seg_offsets, int32_t *kept_count, int64_t *n_dropped)
{
    if (T < 0 || E < 1 || k < 1 || e0 < 0 || E_loc < 1 || e0 + E_loc > E)
        return -1;
    int64_t C = -1;
    if (capacity_factor > 0.0)
        C = (int64_t)floor((double)T * capacity_factor / (double)E);
    *capacity = C;

    int64_t *seen = (int64_t *)calloc((size_t)E_loc, sizeof(int64_t));
    int64_t *rank = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T * k + 1));
    int64_t dropped = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            int e = topk_idx[s];
            if (e < e0 || e >= e0 + E_loc || e >= E) {
                slot_row[s] = -2;
                continue;
            }
            int le = e - e0;
            if (C < 0 || seen[le] < C) {
                rank[s] = seen[le];
                slot_row[s] = 0; /* kept; row assigned below */
            } else {
                slot_row[s] = -1;
                dropped += 1;
            }
            seen[le] += 1;
        }
    }
    seg_offsets[0] = 0;
    for (int le = 0; le < E_loc; ++le) {
        int64_t kept = (C < 0 || seen[le] < C) ? seen[le] : C;
        kept_count[le] = (int32_t)kept;
        seg_offsets[le + 1] = seg_offsets[le] + (int32_t)kept;
    }
    for (int64_t s = 0; s < T * k; ++s) {
        if (slot_row[s] < 0)
            continue;
        int le = topk_idx[s] - e0;
        int32_t row = seg_offsets[le] + (int32_t)rank[s];
        slot_row[s] = row;
        row_src[row] = (int32_t)s;
    }
    *n_dropped = dropped;
    free(seen);
    free(rank);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Expert FFN and combine                                                   */
/* ---------------------------------------------------------------------- */

/* Exact GELU: u * Phi(u) = 0.5 * u * (1 + erf(u / sqrt(2))). */
double oracle_gelu(double u)
{
    return 0.5 * u * (1.0 + erf(u / sqrt(2.0)));
}

/* One expert on one token: out += weight * (W2 . GELU(W1 . x + b1) + b2).
 * W1 is [ffn, d], W2 is [d, ffn] (nn.Linear layout, out x in). */
static void expert_apply(const double *xt, int d, int ffn, int dtype,
                         const void *w1, const void *b1, const void *w2, const void *b2,
                         double weight, double *g, double *out)
{
    for (int f = 0; f < ffn; ++f) {
        double u = 0.0;
        for (int i = 0; i < d; ++i)
            u += elem(w1, dtype, (int64_t)f * d + i) * xt[i];
        if (b1)
            u += elem(b1, dtype, f);
        g[f] = oracle_gelu(u);
    }
    for (int o = 0; o < d; ++o) {
        double v = 0.0;
        for (int f = 0; f < ffn; ++f)
            v += elem(w2, dtype, (int64_t)o * ffn + f) * g[f];
        if (b2)
            v += elem(b2, dtype, o);
        out[o] += weight * v;
    }
}

struct combine_ctx {
    const void *x;
    int dtype;
    int d, k, ffn, e0, E_loc;
    const int64_t *tokens;
    const int32_t *topk_idx, *slot_row;
    const double *topk_w;
    const void *w1, *b1, *w2, *b2, *ws1, *bs1, *ws2, *bs2;
    double *y;
};

static void combine_range(void *p, int64_t i0, int64_t i1)
{
    struct combine_ctx *c = (struct combine_ctx *)p;
    const int d = c->d, ffn = c->ffn, k = c->k;
    double *xt = (double *)malloc(sizeof(double) * (size_t)d);
    double *g = (double *)malloc(sizeof(double) * (size_t)ffn);
    for (int64_t i = i0; i < i1; ++i) {
        int64_t t = c->tokens[i];
        double *yt = c->y + i * d;
        for (int o = 0; o < d; ++o)
            yt[o] = 0.0;
        for (int q = 0; q < d; ++q)
            xt[q] = elem(c->x, c->dtype, t * d + q);
        /* Y = sum over kept selected experts of routing weight * expert output
         * ("MoE Layer Structure"); a dropped selection contributes nothing
         * ("Top-K Routing and Capacity Factor"). */
        for (int j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            if (c->slot_row[s] < 0)
                continue;
            int le = c->topk_idx[s] - c->e0;
            int64_t w1o = (int64_t)le * ffn * d, b1o = (int64_t)le * ffn;
            int64_t w2o = (int64_t)le * d * ffn, b2o = (int64_t)le * d;
            size_t es = c->dtype == ORACLE_DT_BF16 ? 2 : 4;
            expert_apply(xt, d, ffn, c->dtype,
                         (const char *)c->w1 + w1o * es, c->b1 ? (const char *)c->b1 + b1o * es : NULL,
                         (const char *)c->w2 + w2o * es, c->b2 ? (const char *)c->b2 + b2o * es : NULL,
                         c->topk_w[s], g, yt);
        }
        /* Shared expert: every token, weight 1. */
        if (c->ws1)
            expert_apply(xt, d, ffn, c->dtype, c->ws1, c->bs1, c->ws2, c->bs2, 1.0, g, yt);
    }
    free(xt);
    free(g);
}

/* Layer output for the tokens listed in tokens[0..n_tokens).  The selections
 * kept are those with slot_row >= 0 (as produced by oracle_capacity); their
 * expert is topk_idx (global id, local weights indexed by id - e0) and their
 * weight topk_w.  Expert weights: w1 [E_loc, ffn, d], b1 [E_loc, ffn] or NULL,
 * w2 [E_loc, d, ffn], b2 [E_loc, d] or NULL; shared expert ws1 [ffn, d],
 * ws2 [d, ffn] (NULL when absent).  All in the same dtype as x.
 * y is [n_tokens, d]. */
int oracle_combine(const void *x, int dtype, int64_t T, int d, int k, int ffn,
                   const int64_t *tokens, int64_t n_tokens,
                   const int32_t *topk_idx, const double *topk_w, const int32_t *slot_row,
                   int e0, int E_loc,
                   const void *w1, const void *b1, const void *w2, const void *b2,
                   const void *ws1, const void *bs1, const void *ws2, const void *bs2,
                   double *y, int nthreads)
{
    if (T < 0 || d < 1 || k < 1 || ffn < 1 || n_tokens < 0)
        return -1;
    for (int64_t i = 0; i < n_tokens; ++i)
        if (tokens[i] < 0 || tokens[i] >= T)
            return -1;
    struct combine_ctx c = {x, dtype, d, k, ffn, e0, E_loc, tokens, topk_idx, slot_row, topk_w,
                            w1, b1, w2, b2, ws1, bs1, ws2, bs2, y};
    parallel_for(n_tokens, nthreads, combine_range, &c);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Backward: gradients of a scalar loss through the layer                   */
/* ---------------------------------------------------------------------- */

/* d/du GELU(u) = Phi(u) + u * phi(u), with Phi the standard normal CDF and
 * phi its density. */
double oracle_gelu_grad(double u)
{
    const double pi = 3.14159265358979323846;
    return 0.5 * (1.0 + erf(u / sqrt(2.0))) + u * exp(-0.5 * u * u) / sqrt(2.0 * pi);
}

struct bwd_ctx {
    const void *x;
    int dtype;
    int64_t T;
    int d, E, k, ffn, e0, E_loc;
    const float *w_router;
    const double *probs, *topk_w, *f, *dY;
    const int32_t *topk_idx, *slot_row;
    const void *w1, *b1, *w2, *b2, *ws1, *bs1, *ws2, *bs2;
    double g_aux, alpha;
    double *dx, *dlogits;
    /* per-part private accumulators, summed in part order afterwards; NULL
     * when only dx and dlogits of a token subset are wanted */
    int nparts;
    double **acc;
    const int64_t *tokens; /* item i is token tokens[i] (NULL: token i) */
    int64_t n_items;
};

/* sizes of the accumulator block of one part */
static int64_t bwd_acc_size(const struct bwd_ctx *c, int64_t *off)
{
    const int64_t d = c->d, E = c->E, F = c->ffn, L = c->E_loc;
    int64_t o = 0;
    off[0] = o; o += E * d;        /* dW_r */
    off[1] = o; o += E;            /* db_r */
    off[2] = o; o += L * F * d;    /* dW1  */
    off[3] = o; o += L * F;        /* db1  */
    off[4] = o; o += L * d * F;    /* dW2  */
    off[5] = o; o += L * d;        /* db2  */
    off[6] = o; o += c->ws1 ? F * d : 0; /* dWs1 */
    off[7] = o; o += c->ws1 ? F : 0;     /* dbs1 */
    off[8] = o; o += c->ws1 ? d * F : 0; /* dWs2 */
    off[9] = o; o += c->ws1 ? d : 0;     /* dbs2 */
    return o;
}

/* One FFN (W1 [ffn,d], W2 [d,ffn], nn.Linear layout) seen from the output
 * side: Y gets weight * v with v = W2 GELU(W1 x + b1) + b2.  Given dv (the
 * loss gradient at v, already multiplied by the weight), adds dW1, db1, dW2,
 * db2 and dx; returns v . dYt when dYt is given (the gradient of the weight). */
static double ffn_backward(const double *xt, int d, int ffn, int dtype, const void *w1, const void *b1,
                           const void *w2, const void *b2, const double *dv, const double *dYt, double *u,
                           double *g, double *dg, double *dW1, double *db1, double *dW2, double *db2,
                           double *dxt)
{
    for (int q = 0; q < ffn; ++q) {
        double s = 0.0;
        for (int i = 0; i < d; ++i)
            s += elem(w1, dtype, (int64_t)q * d + i) * xt[i];
        if (b1)
            s += elem(b1, dtype, q);
        u[q] = s;
        g[q] = oracle_gelu(s);
    }
    double dw = 0.0;
    if (dYt) {
        for (int o = 0; o < d; ++o) {
            double v = 0.0;
            for (int q = 0; q < ffn; ++q)
                v += elem(w2, dtype, (int64_t)o * ffn + q) * g[q];
            if (b2)
                v += elem(b2, dtype, o);
            dw += dYt[o] * v;
        }
    }
    /* second Linear: dW2 += dv g^T, db2 += dv, dg = W2^T dv (the weight
     * gradients are skipped when dW1 is NULL) */
    for (int q = 0; q < ffn; ++q)
        dg[q] = 0.0;
    for (int o = 0; o < d; ++o) {
        for (int q = 0; q < ffn; ++q) {
            if (dW1)
                dW2[(int64_t)o * ffn + q] += dv[o] * g[q];
            dg[q] += elem(w2, dtype, (int64_t)o * ffn + q) * dv[o];
        }
        if (dW1)
            db2[o] += dv[o];
    }
    /* GELU, then the first Linear: du = dg GELU'(u); dW1 += du x^T, db1 += du,
     * dx += W1^T du */
    for (int q = 0; q < ffn; ++q) {
        const double du = dg[q] * oracle_gelu_grad(u[q]);
        for (int i = 0; i < d; ++i) {
            if (dW1)
                dW1[(int64_t)q * d + i] += du * xt[i];
            dxt[i] += elem(w1, dtype, (int64_t)q * d + i) * du;
        }
        if (dW1)
            db1[q] += du;
    }
    return dw;
}

static void bwd_range(void *p, int64_t t0, int64_t t1)
{
    struct bwd_ctx *c = (struct bwd_ctx *)p;
    const int d = c->d, E = c->E, k = c->k, ffn = c->ffn;
    int64_t off[10];
    bwd_acc_size(c, off);
    /* the part this range belongs to (parallel_for hands out [T p / n,
     * T (p+1) / n) to part p) */
    int part = 0;
    for (int q = 0; q < c->nparts; ++q)
        if (c->n_items * q / c->nparts == t0)
            part = q;
    double *A = c->acc ? c->acc[part] : NULL;
    double *xt = (double *)malloc(sizeof(double) * (size_t)d);
    double *dxt = (double *)malloc(sizeof(double) * (size_t)d);
    double *dv = (double *)malloc(sizeof(double) * (size_t)d);
    double *u = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *g = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *dg = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *dp = (double *)malloc(sizeof(double) * (size_t)E);
    const size_t es = c->dtype == ORACLE_DT_BF16 ? 2 : 4;
    for (int64_t it = t0; it < t1; ++it) {
        const int64_t t = c->tokens ? c->tokens[it] : it;
        const double *dYt = c->dY + t * d;
        const double *pt = c->probs + t * E;
        for (int i = 0; i < d; ++i) {
            xt[i] = elem(c->x, c->dtype, t * d + i);
            dxt[i] = 0.0;
        }
        /* L_aux = alpha sum_e f_e P_e with P_e = mean_t p[t,e]; f counts the
         * selections and has no gradient ("Load Balancing: The Auxiliary
         * Loss"), so dL/dp[t,e] = g_aux alpha f_e / T. */
        for (int e = 0; e < E; ++e)
            dp[e] = c->g_aux * c->alpha * c->f[e] / (double)c->T;
        /* Kept selections: Y_t += w v with w = p[t, e] ("MoE Layer
         * Structure"); dropped and remote selections are not in Y. */
        for (int j = 0; j < k; ++j) {
            const int64_t s = t * k + j;
            if (c->slot_row[s] < 0)
                continue;
            const int e = c->topk_idx[s], le = e - c->e0;
            const double w = c->topk_w[s];
            for (int o = 0; o < d; ++o)
                dv[o] = w * dYt[o];
            const int64_t w1o = (int64_t)le * ffn * d, b1o = (int64_t)le * ffn;
            const int64_t w2o = (int64_t)le * d * ffn, b2o = (int64_t)le * d;
            const double dw = ffn_backward(
                xt, d, ffn, c->dtype, (const char *)c->w1 + w1o * es, c->b1 ? (const char *)c->b1 + b1o * es : NULL,
                (const char *)c->w2 + w2o * es, c->b2 ? (const char *)c->b2 + b2o * es : NULL, dv, dYt, u, g, dg,
                A ? A + off[2] + w1o : NULL, A ? A + off[3] + b1o : NULL, A ? A + off[4] + w2o : NULL,
                A ? A + off[5] + b2o : NULL, dxt);
            dp[e] += dw;
        }
        /* Router: w = softmax(logits)[e]; dl_i = p_i (dp_i - sum_e p_e dp_e). */
        double sdot = 0.0;
        for (int e = 0; e < E; ++e)
            sdot += pt[e] * dp[e];
        for (int e = 0; e < E; ++e) {
            const double dl = pt[e] * (dp[e] - sdot);
            if (c->dlogits)
                c->dlogits[it * E + e] = dl;
            if (A)
                A[off[1] + e] += dl;
            for (int i = 0; i < d; ++i) {
                if (A)
                    A[off[0] + (int64_t)e * d + i] += dl * xt[i];
                dxt[i] += (double)c->w_router[(int64_t)e * d + i] * dl;
            }
        }
        /* Shared expert: weight 1 on every token. */
        if (c->ws1)
            ffn_backward(xt, d, ffn, c->dtype, c->ws1, c->bs1, c->ws2, c->bs2, dYt, NULL, u, g, dg,
                         A ? A + off[6] : NULL, A ? A + off[7] : NULL, A ? A + off[8] : NULL, A ? A + off[9] : NULL,
                         dxt);
        for (int i = 0; i < d; ++i)
            c->dx[it * d + i] = dxt[i];
    }
    free(xt);
    free(dxt);
    free(dv);
    free(u);
    free(g);
    free(dg);
    free(dp);
}

/* Gradients of a scalar loss with dL/dY = dY [T, d] (float64) and
 * dL/dL_aux = g_aux, through the layer whose forward made topk_idx,
 * topk_w (= probs at the selection), slot_row (oracle_capacity) and f.
 * probs [T, E] are the router's softmax probabilities.  Selection (top-k,
 * capacity) is piecewise constant and has no gradient.  Outputs (float64,
 * all required except the shared-expert ones when ws1 is NULL and dlogits):
 * dx [T,d], dW_r [E,d], db_r [E], dW1 [E_loc,ffn,d], db1 [E_loc,ffn],
 * dW2 [E_loc,d,ffn], db2 [E_loc,d], dWs1 [ffn,d], dbs1 [ffn], dWs2 [d,ffn],
 * dbs2 [d], dlogits [T,E]. */
int oracle_backward(const void *x, int dtype, int64_t T, int d, int E, int k, int ffn, const float *w_router,
                    const double *probs, const int32_t *topk_idx, const double *topk_w, const int32_t *slot_row,
                    const double *f, double alpha, double g_aux, int e0, int E_loc, const void *w1, const void *b1,
                    const void *w2, const void *b2, const void *ws1, const void *bs1, const void *ws2,
                    const void *bs2, const double *dY, double *dx, double *dW_r, double *db_r, double *dW1,
                    double *db1, double *dW2, double *db2, double *dWs1, double *dbs1, double *dWs2, double *dbs2,
                    double *dlogits, int nthreads)
{
    if (T < 1 || d < 1 || E < 1 || k < 1 || ffn < 1 || e0 < 0 || E_loc < 1 || e0 + E_loc > E)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > T)
        nthreads = (int)T;
    struct bwd_ctx c = {x, dtype, T, d, E, k, ffn, e0, E_loc, w_router, probs, topk_w, f, dY, topk_idx, slot_row,
                        w1, b1, w2, b2, ws1, bs1, ws2, bs2, g_aux, alpha, dx, dlogits, nthreads, NULL, NULL, T};
    int64_t off[10];
    const int64_t n = bwd_acc_size(&c, off);
    c.acc = (double **)malloc(sizeof(double *) * (size_t)nthreads);
    for (int p = 0; p < nthreads; ++p) {
        c.acc[p] = (double *)calloc((size_t)n, sizeof(double));
        if (!c.acc[p])
            return -2;
    }
    /* one contiguous token range per part, so each accumulator is private */
    parallel_for(T, nthreads, bwd_range, &c);
    /* fixed-order sum of the parts */
    double *outs[10] = {dW_r, db_r, dW1, db1, dW2, db2, dWs1, dbs1, dWs2, dbs2};
    for (int q = 0; q < 10; ++q) {
        const int64_t len = (q < 9 ? off[q + 1] : n) - off[q];
        if (!outs[q] || len == 0)
            continue;
        for (int64_t i = 0; i < len; ++i) {
            double s = 0.0;
            for (int p = 0; p < nthreads; ++p)
                s += c.acc[p][off[q] + i];
            outs[q][i] = s;
        }
    }
    for (int p = 0; p < nthreads; ++p)
        free(c.acc[p]);
    free(c.acc);
    return 0;
}

/* dx and dlogits of the tokens tokens[0..n_tokens) only (rows i of dx
 * [n_tokens, d] and dlogits [n_tokens, E]), with the same arithmetic as
 * oracle_backward; no weight gradients.  Arguments otherwise as there. */
int oracle_backward_tokens(const void *x, int dtype, int64_t T, int d, int E, int k, int ffn, const float *w_router,
                           const double *probs, const int32_t *topk_idx, const double *topk_w,
                           const int32_t *slot_row, const double *f, double alpha, double g_aux, int e0, int E_loc,
                           const void *w1, const void *b1, const void *w2, const void *b2, const void *ws1,
                           const void *bs1, const void *ws2, const void *bs2, const double *dY,
                           const int64_t *tokens, int64_t n_tokens, double *dx, double *dlogits, int nthreads)
{
    if (T < 1 || d < 1 || E < 1 || k < 1 || ffn < 1 || e0 < 0 || E_loc < 1 || e0 + E_loc > E || n_tokens < 0)
        return -1;
    for (int64_t i = 0; i < n_tokens; ++i)
        if (tokens[i] < 0 || tokens[i] >= T)
            return -1;
    if (n_tokens == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > n_tokens)
        nthreads = (int)n_tokens;
    struct bwd_ctx c = {x, dtype, T, d, E, k, ffn, e0, E_loc, w_router, probs, topk_w, f, dY, topk_idx, slot_row,
                        w1, b1, w2, b2, ws1, bs1, ws2, bs2, g_aux, alpha, dx, dlogits, nthreads, NULL, tokens,
                        n_tokens};
    parallel_for(n_tokens, nthreads, bwd_range, &c);
    return 0;
}

/* Columns of one FFN's weight gradients, from the definition restricted to
 * feature q of the hidden layer.  The FFN (w1 [ffn,d], b1 [ffn] or NULL,
 * w2 [d,ffn], nn.Linear layout, dtype of x) sees rows r = 0..n_rows-1:
 * token tok[r] with output weight wt[r] (Y_t += wt v).  For each q = qs[j]:
 *   u = w1[q,:] . x_t + b1[q],  dg = sum_o w2[o,q] dY[t,o],
 *   du = wt dg GELU'(u)
 *   dW1_row[j, :] = sum_r du x_t,   db1[j] = sum_r du,
 *   dW2_col[j, o] = sum_r dY[t,o] wt GELU(u)    (column q of dW2)
 * and db2 [d] = sum_r wt dY[t, :] (if not NULL).  Sums run in row order. */
struct col_ctx {
    const void *x, *w1, *b1, *w2;
    int dtype, d, ffn;
    const int64_t *tok;
    const double *wt, *dY;
    int64_t n_rows;
    const int32_t *qs;
    double *dW1_row, *db1, *dW2_col;
};

static void col_range(void *p, int64_t j0, int64_t j1)
{
    struct col_ctx *c = (struct col_ctx *)p;
    const int d = c->d, F = c->ffn;
    for (int64_t j = j0; j < j1; ++j) {
        const int q = c->qs[j];
        double *rw = c->dW1_row + j * d, *cw = c->dW2_col + j * d;
        double sb = 0.0;
        for (int i = 0; i < d; ++i)
            rw[i] = cw[i] = 0.0;
        for (int64_t r = 0; r < c->n_rows; ++r) {
            const int64_t t = c->tok[r];
            double u = c->b1 ? elem(c->b1, c->dtype, q) : 0.0;
            for (int i = 0; i < d; ++i)
                u += elem(c->w1, c->dtype, (int64_t)q * d + i) * elem(c->x, c->dtype, t * d + i);
            double dg = 0.0;
            for (int o = 0; o < d; ++o)
                dg += elem(c->w2, c->dtype, (int64_t)o * F + q) * c->dY[t * d + o];
            const double du = c->wt[r] * dg * oracle_gelu_grad(u);
            const double gw = c->wt[r] * oracle_gelu(u);
            for (int i = 0; i < d; ++i) {
                rw[i] += du * elem(c->x, c->dtype, t * d + i);
                cw[i] += c->dY[t * d + i] * gw;
            }
            sb += du;
        }
        c->db1[j] = sb;
    }
}

int oracle_ffn_grad_columns(const void *x, int dtype, int64_t T, int d, int ffn, const void *w1, const void *b1,
                            const void *w2, const int64_t *tok, const double *wt, int64_t n_rows, const double *dY,
                            const int32_t *qs, int nq, double *dW1_row, double *db1, double *dW2_col, double *db2,
                            int nthreads)
{
    if (T < 0 || d < 1 || ffn < 1 || n_rows < 0 || nq < 0)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (tok[r] < 0 || tok[r] >= T)
            return -1;
    for (int j = 0; j < nq; ++j)
        if (qs[j] < 0 || qs[j] >= ffn)
            return -1;
    if (db2) {
        for (int o = 0; o < d; ++o) {
            double s = 0.0;
            for (int64_t r = 0; r < n_rows; ++r)
                s += wt[r] * dY[tok[r] * d + o];
            db2[o] = s;
        }
    }
    if (nq == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nq)
        nthreads = nq;
    struct col_ctx c = {x, w1, b1, w2, dtype, d, ffn, tok, wt, dY, n_rows, qs, dW1_row, db1, dW2_col};
    parallel_for(nq, nthreads, col_range, &c);
    return 0;
}
