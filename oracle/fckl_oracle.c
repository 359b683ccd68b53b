/*
 * fckl_oracle.c -- CPU oracle for the offline top-K distillation KL loss.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously correct
 * statement of what the fused chunked loss computes.  It is used by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg, and by
 * nothing else: the product library never links, loads or calls it, and it
 * shares no code, header, table or helper with the GPU library.
 *
 * What is computed (all arithmetic in IEEE double):
 *
 *   The teacher cache holds, per token i, K logits tl[i,k] and their vocabulary
 *   indices idx[i,k] ("Preparing Offline Top-K Logits", getaibook.com; "Breaking
 *   the Bottleneck with Offline Caching and Chunked Loss", axbrief.com: the top
 *   100 logits are extracted once and stored).
 *
 *   1. Teacher distribution over the K cached entries, at temperature T:
 *        lp[k] = tl[k]/T - log sum_j exp(tl[j]/T),   p[k] = exp(lp[k]).
 *      The pages do not say how the mass outside the top-K is handled; the
 *      reading taken here renormalises over the K cached entries (no tail bucket).
 *   2. Student logits over the full vocabulary: the output projection is part of
 *      the loss ("What actually changed?", calcaas.com: the fused loss folds the
 *      model's output projection into the loss):
 *        z[i,v] = sum_j h[i,j] * W[v,j].
 *   3. lse[i] = log sum_v exp(z[i,v]/T)   (natural log, max-shifted).
 *   4. log q[i,k] = z[i,idx[i,k]]/T - lse[i].
 *   5. loss[i] = T^2 * sum_k p[k] * (lp[k] - log q[i,k])   -- forward KL(p || q),
 *      the KL divergence the pages name ("Configuring Fused Chunked KL Loss",
 *      getaibook.com) taken from the teacher's cached distribution to the student's.
 *      The reported loss is the mean of loss[i] over the N tokens.
 *   6. Gradient of (grad_scale * mean loss) with respect to z:
 *        g[i,v] = grad_scale * (T/N) * ( (sum_k p[k]) * exp(z[i,v]/T - lse[i])
 *                                        - sum_k p[k] * [idx[i,k] == v] ).
 *   7. dH[i,:] = sum_v g[i,v] * W[v,:];   dW[v,:] = sum_i g[i,v] * h[i,:].
 *
 * The chunking of the method changes where and when these numbers are formed,
 * not their values, so the oracle does not chunk ("Breaking the Bottleneck ...",
 * axbrief.com: one slice of the sequence at a time, then discarded).
 *
 * Token masks and per-token weights (the weighted reduction below) change only the
 * reduction: with weights w[i] >= 0 the reported loss is
 *      sum_i w[i] loss[i] / sum_i w[i]     (0 when every weight is 0),
 * a masked token being one with w[i] = 0, and step 6 scales row i by
 * grad_scale * T * w[i] / sum_j w[j] instead of grad_scale * T / N.  All weights 1
 * give the plain mean.
 *
 * Inputs are double arrays, row-major: h[N*H], W[V*H], idx[N*K] (int32),
 * tl[N*K].  A row list (rows, nrows) selects which tokens are evaluated; rows ==
 * NULL means all N tokens in order.  Return value 0 on success, negative on a
 * rejected argument (see the ORACLE_E* codes below); outputs are then untouched.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EARG (-1)   /* bad sizes, T <= 0, NULL pointers */
#define ORACLE_EIDX (-2)   /* a cached index outside [0, V) */
#define ORACLE_EMEM (-3)   /* host allocation failed */

static int check_args(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                      const double *h, const double *W, const int32_t *idx,
                      const double *tl, int64_t nrows, const int64_t *rows)
{
    if (N < 0 || H <= 0 || V <= 0 || K <= 0 || !(T > 0.0) || isinf(T))
        return ORACLE_EARG;
    if (!h || !W || !idx || !tl || nrows < 0)
        return ORACLE_EARG;
    if (!rows && nrows != N)
        return ORACLE_EARG;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= N)
            return ORACLE_EARG;
        for (int64_t k = 0; k < K; ++k) {
            int32_t v = idx[i * K + k];
            if (v < 0 || (int64_t)v >= V)
                return ORACLE_EIDX;
        }
    }
    return ORACLE_OK;
}

/* Step 1: teacher probabilities p and log-probabilities lp over the K entries. */
static void teacher_distribution(int64_t K, double T, const double *tl, double *p, double *lp)
{
    double m = -INFINITY;
    for (int64_t k = 0; k < K; ++k)
        if (tl[k] / T > m)
            m = tl[k] / T;
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += exp(tl[k] / T - m);
    double log_norm = m + log(s);
    for (int64_t k = 0; k < K; ++k) {
        lp[k] = tl[k] / T - log_norm;
        p[k] = exp(lp[k]);
    }
}

/* Step 2: student logits of one token over the whole vocabulary. */
static void student_logits(int64_t H, int64_t V, const double *h_row, const double *W, double *z)
{
    for (int64_t v = 0; v < V; ++v) {
        const double *w = W + v * H;
        double acc = 0.0;
        for (int64_t j = 0; j < H; ++j)
            acc += h_row[j] * w[j];
        z[v] = acc;
    }
}

/* Step 3: log sum_v exp(z[v]/T), shifted by the maximum. */
static double logsumexp_over_vocab(int64_t V, double T, const double *z)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v)
        if (z[v] / T > m)
            m = z[v] / T;
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v)
        s += exp(z[v] / T - m);
    return m + log(s);
}

/*
 * Forward: per-token loss (steps 1-5) and lse (step 3) for the selected rows.
 * loss_out[r], lse_out[r] refer to row rows[r] (or r).  Either output may be NULL.
 */
int fckl_oracle_forward(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                        const double *h, const double *W, const int32_t *idx,
                        const double *tl, int64_t nrows, const int64_t *rows,
                        double *loss_out, double *lse_out)
{
    int rc = check_args(N, H, V, K, T, h, W, idx, tl, nrows, rows);
    if (rc)
        return rc;
    int failed = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
        double *p = (double *)malloc(sizeof(double) * (size_t)K);
        double *lp = (double *)malloc(sizeof(double) * (size_t)K);
        int have = (z && p && lp);
        if (!have) {
#pragma omp atomic write
            failed = 1;
        }
        /* Every thread reaches the worksharing loop; one without buffers skips its rows. */
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!have)
                continue;
            {
                int64_t i = rows ? rows[r] : r;
                teacher_distribution(K, T, tl + i * K, p, lp);
                student_logits(H, V, h + i * H, W, z);
                double lse = logsumexp_over_vocab(V, T, z);
                double kl = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double log_q = z[idx[i * K + k]] / T - lse;
                    kl += p[k] * (lp[k] - log_q);
                }
                if (loss_out)
                    loss_out[r] = T * T * kl;
                if (lse_out)
                    lse_out[r] = lse;
            }
        }
        free(z);
        free(p);
        free(lp);
    }
    return failed ? ORACLE_EMEM : ORACLE_OK;
}

/* Mean of the per-token loss over all N tokens (the reduction of step 5). */
int fckl_oracle_loss_mean(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                          const double *h, const double *W, const int32_t *idx,
                          const double *tl, double *mean_out)
{
    if (N <= 0 || !mean_out)
        return ORACLE_EARG;
    double *loss = (double *)malloc(sizeof(double) * (size_t)N);
    if (!loss)
        return ORACLE_EMEM;
    int rc = fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, N, NULL, loss, NULL);
    if (rc == ORACLE_OK) {
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i)
            s += loss[i];
        *mean_out = s / (double)N;
    }
    free(loss);
    return rc;
}

/*
 * Steps 6-7 for the selected rows, row r's gradient scaled by row_scale[r]:
 *   g[r,v] = row_scale[r] * ( (sum_k p[k]) exp(z[v]/T - lse) - sum_k p[k] [idx[k] == v] ).
 * dH_out[r*H + j] is the gradient for row rows[r]; dW_out[V*H] receives the sum over
 * the selected rows only (it is overwritten).  Either output may be NULL.
 */
static int backward_rows(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                         const double *h, const double *W, const int32_t *idx,
                         const double *tl, const double *row_scale,
                         int64_t nrows, const int64_t *rows,
                         double *dH_out, double *dW_out)
{
    (void)N;
    /* g for every selected row, held whole: nrows * V doubles. */
    double *g = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * (size_t)V);
    if (!g)
        return ORACLE_EMEM;
    int failed = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
        double *p = (double *)malloc(sizeof(double) * (size_t)K);
        double *lp = (double *)malloc(sizeof(double) * (size_t)K);
        int have = (z && p && lp);
        if (!have) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!have)
                continue;
            {
                int64_t i = rows ? rows[r] : r;
                const double scale = row_scale[r];
                teacher_distribution(K, T, tl + i * K, p, lp);
                student_logits(H, V, h + i * H, W, z);
                double lse = logsumexp_over_vocab(V, T, z);
                double psum = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    psum += p[k];
                double *gr = g + r * V;
                for (int64_t v = 0; v < V; ++v)
                    gr[v] = scale * psum * exp(z[v] / T - lse);
                for (int64_t k = 0; k < K; ++k)
                    gr[idx[i * K + k]] -= scale * p[k];
            }
        }
        free(z);
        free(p);
        free(lp);
    }
    if (failed) {
        free(g);
        return ORACLE_EMEM;
    }
    if (dH_out) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            double *out = dH_out + r * H;
            for (int64_t j = 0; j < H; ++j)
                out[j] = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                double gv = g[r * V + v];
                const double *w = W + v * H;
                for (int64_t j = 0; j < H; ++j)
                    out[j] += gv * w[j];
            }
        }
    }
    if (dW_out) {
        /* Each vocabulary row is owned by one thread: no shared accumulation. */
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) {
            double *out = dW_out + v * H;
            for (int64_t j = 0; j < H; ++j)
                out[j] = 0.0;
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows ? rows[r] : r;
                double gv = g[r * V + v];
                const double *hr = h + i * H;
                for (int64_t j = 0; j < H; ++j)
                    out[j] += gv * hr[j];
            }
        }
    }
    free(g);
    return ORACLE_OK;
}

/*
 * Backward (steps 6-7) of grad_scale * (1/n_norm) * sum over the selected rows
 * of loss[i].  With rows == NULL and n_norm == N this is the gradient of
 * grad_scale * mean loss.
 */
int fckl_oracle_backward(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                         const double *h, const double *W, const int32_t *idx,
                         const double *tl, double grad_scale, int64_t n_norm,
                         int64_t nrows, const int64_t *rows,
                         double *dH_out, double *dW_out)
{
    int rc = check_args(N, H, V, K, T, h, W, idx, tl, nrows, rows);
    if (rc)
        return rc;
    if (n_norm <= 0)
        return ORACLE_EARG;
    double *scale = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    if (!scale)
        return ORACLE_EMEM;
    for (int64_t r = 0; r < nrows; ++r)
        scale[r] = grad_scale * T / (double)n_norm;
    rc = backward_rows(N, H, V, K, T, h, W, idx, tl, scale, nrows, rows, dH_out, dW_out);
    free(scale);
    return rc;
}

/* sum_i w[i] over all N tokens; ORACLE_EARG for a negative or non-finite weight. */
static int weight_sum(int64_t N, const double *w, double *sum)
{
    if (!w)
        return ORACLE_EARG;
    double s = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        if (!(w[i] >= 0.0) || isinf(w[i]))
            return ORACLE_EARG;
        s += w[i];
    }
    *sum = s;
    return ORACLE_OK;
}

/* Weighted mean of the per-token loss: sum_i w[i] loss[i] / sum_i w[i] (0 if all w are 0). */
int fckl_oracle_weighted_mean(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                              const double *h, const double *W, const int32_t *idx,
                              const double *tl, const double *w, double *mean_out)
{
    if (N <= 0 || !mean_out)
        return ORACLE_EARG;
    double wsum = 0.0;
    int rc = weight_sum(N, w, &wsum);
    if (rc)
        return rc;
    double *loss = (double *)malloc(sizeof(double) * (size_t)N);
    if (!loss)
        return ORACLE_EMEM;
    rc = fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, N, NULL, loss, NULL);
    if (rc == ORACLE_OK) {
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i)
            s += w[i] * loss[i];
        *mean_out = wsum > 0.0 ? s / wsum : 0.0;
    }
    free(loss);
    return rc;
}

/*
 * Gradient of grad_scale * (weighted mean loss) for the selected rows: row i is
 * scaled by grad_scale * T * w[i] / sum_j w[j] (the sum over all N tokens), and by 0
 * when every weight is 0.
 */
int fckl_oracle_weighted_backward(int64_t N, int64_t H, int64_t V, int64_t K, double T,
                                  const double *h, const double *W, const int32_t *idx,
                                  const double *tl, const double *w, double grad_scale,
                                  int64_t nrows, const int64_t *rows,
                                  double *dH_out, double *dW_out)
{
    int rc = check_args(N, H, V, K, T, h, W, idx, tl, nrows, rows);
    if (rc)
        return rc;
    double wsum = 0.0;
    rc = weight_sum(N, w, &wsum);
    if (rc)
        return rc;
    double *scale = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    if (!scale)
        return ORACLE_EMEM;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        scale[r] = wsum > 0.0 ? grad_scale * T * w[i] / wsum : 0.0;
    }
    rc = backward_rows(N, H, V, K, T, h, W, idx, tl, scale, nrows, rows, dH_out, dW_out);
    free(scale);
    return rc;
}

/*
 * Teacher-side top-K extraction: the cache the loss reads.  The pages describe the
 * teacher's top logits (100, or 10) and their vocabulary indices being extracted once
 * per position and stored ("Preparing Offline Top-K Logits", getaibook.com;
 * "Breaking the Bottleneck with Offline Caching and Chunked Loss", axbrief.com).
 * For each token i: z[v] = sum_j h[i,j] W[v,j] over the whole vocabulary, then the K
 * entries with the largest z, in descending order of z; equal values are ordered by
 * the smaller index first, which makes the result unique.
 *   idx_out[N*K] (int32), val_out[N*K] (the z of each entry).
 */
typedef struct {
    double z;
    int32_t v;
} ranked_logit;

static int rank_before(const ranked_logit *a, const ranked_logit *b)
{
    return a->z > b->z || (a->z == b->z && a->v < b->v);
}

int fckl_oracle_topk(int64_t N, int64_t H, int64_t V, int64_t K, const double *h, const double *W,
                     int32_t *idx_out, double *val_out)
{
    if (N < 0 || H <= 0 || V <= 0 || K <= 0 || K > V || !h || !W || !idx_out || !val_out)
        return ORACLE_EARG;
    int failed = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
        ranked_logit *best = (ranked_logit *)malloc(sizeof(ranked_logit) * (size_t)K);
        int have = (z && best);
        if (!have) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < N; ++i) {
            if (!have)
                continue;
            student_logits(H, V, h + i * H, W, z);
            /* insertion into a sorted list of the K best seen so far */
            int64_t n = 0;
            for (int64_t v = 0; v < V; ++v) {
                ranked_logit c = {z[v], (int32_t)v};
                if (n == K && !rank_before(&c, &best[K - 1]))
                    continue;
                int64_t at = n < K ? n : K - 1;
                while (at > 0 && rank_before(&c, &best[at - 1])) {
                    best[at] = best[at - 1];
                    --at;
                }
                best[at] = c;
                if (n < K)
                    ++n;
            }
            for (int64_t k = 0; k < K; ++k) {
                idx_out[i * K + k] = best[k].v;
                val_out[i * K + k] = best[k].z;
            }
        }
        free(z);
        free(best);
    }
    return failed ? ORACLE_EMEM : ORACLE_OK;
}

/*
 * Online distillation against the full teacher distribution (the variant the pages
 * compare the cached top-K teacher with: the teacher's full vocabulary distribution,
 * computed next to the student's, "The Distillation Bottleneck", getaibook.com; the
 * teacher forward on the fly, "The 250GB VRAM Wall in Long-Context Distillation",
 * axbrief.com).  The teacher's hidden states ht[N*Ht] and LM head Wt[V*Ht] are inputs:
 *   p = softmax(zt / T) over the whole vocabulary, zt[v] = ht . Wt[v]
 *   q = softmax(zs / T),                            zs[v] = hs . Ws[v]
 *   loss[i] = T^2 * sum_v p[v] (log p[v] - log q[v])
 * reduced as the weighted mean (w == NULL: all weights 1), and the gradient of
 * grad_scale * mean with respect to the student:
 *   g[i,v] = grad_scale * T * w[i] / sum_j w[j] * (q[v] - p[v]);  dH = g Ws,  dW = g^T hs.
 * lse_out[i] = log sum_v exp(zs[v] / T).  Any of the outputs may be NULL.
 */
int fckl_oracle_full(int64_t N, int64_t Hs, int64_t Ht, int64_t V, double T,
                     const double *hs, const double *Ws, const double *ht, const double *Wt,
                     const double *w, double grad_scale,
                     double *loss_out, double *lse_out, double *mean_out,
                     double *dH_out, double *dW_out)
{
    if (N <= 0 || Hs <= 0 || Ht <= 0 || V <= 0 || !(T > 0.0) || isinf(T) || !hs || !Ws || !ht || !Wt)
        return ORACLE_EARG;
    double wsum = (double)N;
    if (w && weight_sum(N, w, &wsum))
        return ORACLE_EARG;
    double *g = (double *)malloc(sizeof(double) * (size_t)N * (size_t)V);
    double *loss = (double *)malloc(sizeof(double) * (size_t)N);
    if (!g || !loss) {
        free(g);
        free(loss);
        return ORACLE_EMEM;
    }
    int failed = 0;
#pragma omp parallel
    {
        double *zs = (double *)malloc(sizeof(double) * (size_t)V);
        double *zt = (double *)malloc(sizeof(double) * (size_t)V);
        int have = (zs && zt);
        if (!have) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < N; ++i) {
            if (!have)
                continue;
            student_logits(Ht, V, ht + i * Ht, Wt, zt);
            student_logits(Hs, V, hs + i * Hs, Ws, zs);
            const double lt = logsumexp_over_vocab(V, T, zt);
            const double ls = logsumexp_over_vocab(V, T, zs);
            const double scale = wsum > 0.0 ? grad_scale * T * (w ? w[i] : 1.0) / wsum : 0.0;
            double kl = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                const double log_p = zt[v] / T - lt, log_q = zs[v] / T - ls;
                const double p = exp(log_p);
                kl += p * (log_p - log_q);
                g[i * V + v] = scale * (exp(log_q) - p);
            }
            loss[i] = T * T * kl;
            if (loss_out)
                loss_out[i] = loss[i];
            if (lse_out)
                lse_out[i] = ls;
        }
        free(zs);
        free(zt);
    }
    if (!failed && mean_out) {
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i)
            s += (w ? w[i] : 1.0) * loss[i];
        *mean_out = wsum > 0.0 ? s / wsum : 0.0;
    }
    if (!failed && dH_out) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < N; ++i) {
            double *out = dH_out + i * Hs;
            for (int64_t j = 0; j < Hs; ++j)
                out[j] = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                const double gv = g[i * V + v];
                const double *wr = Ws + v * Hs;
                for (int64_t j = 0; j < Hs; ++j)
                    out[j] += gv * wr[j];
            }
        }
    }
    if (!failed && dW_out) {
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) {
            double *out = dW_out + v * Hs;
            for (int64_t j = 0; j < Hs; ++j)
                out[j] = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                const double gv = g[i * V + v];
                const double *hr = hs + i * Hs;
                for (int64_t j = 0; j < Hs; ++j)
                    out[j] += gv * hr[j];
            }
        }
    }
    free(g);
    free(loss);
    return failed ? ORACLE_EMEM : ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int fckl_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
