/*
 * Sanitizer driver for the CPU oracle (test infrastructure): calls every oracle entry
 * point on small seeded inputs, with rows subsets, NULL outputs and rejected
 * arguments, so that AddressSanitizer and UndefinedBehaviorSanitizer see every path.
 * Checks only what holds for any input: status codes, finite results, loss >= 0,
 * sum over the vocabulary of dW = 0.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int fckl_oracle_forward(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *,
                        const int32_t *, const double *, int64_t, const int64_t *, double *, double *);
int fckl_oracle_loss_mean(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *,
                          const int32_t *, const double *, double *);
int fckl_oracle_backward(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *,
                         const int32_t *, const double *, double, int64_t, int64_t, const int64_t *, double *,
                         double *);
int fckl_oracle_weighted_mean(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *,
                              const int32_t *, const double *, const double *, double *);
int fckl_oracle_weighted_backward(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *,
                                  const int32_t *, const double *, const double *, double, int64_t,
                                  const int64_t *, double *, double *);
int fckl_oracle_topk(int64_t, int64_t, int64_t, int64_t, const double *, const double *, int32_t *, double *);
int fckl_oracle_full(int64_t, int64_t, int64_t, int64_t, double, const double *, const double *, const double *,
                     const double *, const double *, double, double *, double *, double *, double *, double *);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}
static double *draw(int64_t n, double scale)
{
    double *x = malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i)
        x[i] = scale * (2.0 * uniform() - 1.0);
    return x;
}
static int failures = 0;
#define CHECK(cond)                                                                                           \
    do {                                                                                                      \
        if (!(cond)) {                                                                                        \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);                                \
            ++failures;                                                                                       \
        }                                                                                                     \
    } while (0)

static void run_shape(int64_t N, int64_t H, int64_t V, int64_t K, double T)
{
    double *h = draw(N * H, 1.0), *W = draw(V * H, 0.5), *tl = draw(N * K, 2.0);
    int32_t *idx = malloc((size_t)(N * K) * sizeof(int32_t));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t k = 0; k < K; ++k)
            idx[i * K + k] = (int32_t)((i * 7 + k * 13) % V);   /* distinct when K <= V and gcd(13, V) = 1 */
    /* per-row outputs hold nrows entries: N, or the 2 of the rows subset below */
    const int64_t nout = N > 2 ? N : 2;
    double *loss = malloc((size_t)nout * sizeof(double)), *lse = malloc((size_t)nout * sizeof(double));
    double *dH = malloc((size_t)(nout * H) * sizeof(double)), *dW = malloc((size_t)(V * H) * sizeof(double));
    double *w = draw(N, 1.0), mean = 0.0;
    for (int64_t i = 0; i < N; ++i)
        w[i] = fabs(w[i]);
    CHECK(fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, N, NULL, loss, lse) == 0);
    for (int64_t i = 0; i < N; ++i)
        CHECK(isfinite(loss[i]) && loss[i] >= -1e-12 && isfinite(lse[i]));
    CHECK(fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, N, NULL, NULL, lse) == 0);
    int64_t rows[2] = {N - 1, 0};
    CHECK(fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, 2, rows, loss, NULL) == 0);
    CHECK(fckl_oracle_loss_mean(N, H, V, K, T, h, W, idx, tl, &mean) == 0 && isfinite(mean));
    CHECK(fckl_oracle_backward(N, H, V, K, T, h, W, idx, tl, 1.5, N, N, NULL, dH, dW) == 0);
    for (int64_t j = 0; j < H; ++j) {
        double s = 0.0, a = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            s += dW[v * H + j];
            a += fabs(dW[v * H + j]);
        }
        CHECK(fabs(s) <= 1e-10 * (a + 1e-300));
    }
    CHECK(fckl_oracle_backward(N, H, V, K, T, h, W, idx, tl, 1.0, N, 2, rows, dH, NULL) == 0);
    CHECK(fckl_oracle_weighted_mean(N, H, V, K, T, h, W, idx, tl, w, &mean) == 0 && isfinite(mean));
    CHECK(fckl_oracle_weighted_backward(N, H, V, K, T, h, W, idx, tl, w, 0.5, N, NULL, dH, dW) == 0);
    CHECK(fckl_oracle_weighted_backward(N, H, V, K, T, h, W, idx, tl, w, 0.5, 2, rows, NULL, dW) == 0);
    int32_t *ti = malloc((size_t)(N * K) * sizeof(int32_t));
    double *tv = malloc((size_t)(N * K) * sizeof(double));
    CHECK(fckl_oracle_topk(N, H, V, K, h, W, ti, tv) == 0);
    for (int64_t i = 0; i < N; ++i)
        for (int64_t k = 1; k < K; ++k)
            CHECK(tv[i * K + k - 1] >= tv[i * K + k]);
    double *ht = draw(N * (H + 3), 1.0), *Wt = draw(V * (H + 3), 0.5);
    CHECK(fckl_oracle_full(N, H, H + 3, V, T, h, W, ht, Wt, w, 2.0, loss, lse, &mean, dH, dW) == 0);
    for (int64_t i = 0; i < N; ++i)
        CHECK(isfinite(loss[i]) && loss[i] >= -1e-12);
    CHECK(fckl_oracle_full(N, H, H + 3, V, T, h, W, ht, Wt, NULL, 1.0, NULL, NULL, NULL, dH, NULL) == 0);
    /* rejected arguments: outputs untouched, an error code */
    idx[0] = (int32_t)V;
    CHECK(fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, N, NULL, loss, lse) != 0);
    idx[0] = -1;
    CHECK(fckl_oracle_backward(N, H, V, K, T, h, W, idx, tl, 1.0, N, N, NULL, dH, dW) != 0);
    idx[0] = 0;
    CHECK(fckl_oracle_forward(N, H, V, K, -1.0, h, W, idx, tl, N, NULL, loss, lse) != 0);
    int64_t bad_rows[1] = {N};
    CHECK(fckl_oracle_forward(N, H, V, K, T, h, W, idx, tl, 1, bad_rows, loss, lse) != 0);
    CHECK(fckl_oracle_topk(N, H, V, V + 1, h, W, ti, tv) != 0);
    CHECK(fckl_oracle_full(N, H, H + 3, V, 0.0, h, W, ht, Wt, NULL, 1.0, loss, lse, &mean, dH, dW) != 0);
    w[0] = -1.0;
    CHECK(fckl_oracle_weighted_mean(N, H, V, K, T, h, W, idx, tl, w, &mean) != 0);
    free(h); free(W); free(tl); free(idx); free(loss); free(lse); free(dH); free(dW); free(w);
    free(ti); free(tv); free(ht); free(Wt);
}

int main(void)
{
    run_shape(5, 7, 37, 4, 1.3);
    run_shape(1, 8, 16, 16, 0.5);
    run_shape(9, 3, 41, 1, 2.0);
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle driver ok\n");
    return failures ? 1 : 0;
}
