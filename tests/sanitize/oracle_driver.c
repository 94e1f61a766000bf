/*
 * Drives every entry point of oracle/pisa_oracle.c on small inputs (ragged
 * lengths, causal and not, grouped heads) for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use of freed memory or
 * undefined operation in the oracle aborts this program with a report.
 * Test infrastructure (tests/test_sanitizers.py builds and runs it).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_levels(int64_t N, int C, int g, int64_t *M);
void orc_build_pyramid(const float *K, int B, int64_t N_alloc, int64_t N, int H, int d, int C, int g,
                       double *pyr, const int64_t *off);
int orc_route_scored(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                     const float *K, const double *pyr, const int64_t *off, int B, int64_t N_alloc,
                     int64_t N, int H, int H_q, int d, int C, int g, int K_top, int causal,
                     int score_kind, int32_t *idx, double *score, double *gap, int32_t *trace,
                     int nthreads);
int orc_route_reach(const float *Q, const int64_t *item_b, const int64_t *item_t,
                    const int32_t *item_h, int64_t n_items, const float *K, const double *pyr,
                    const int64_t *off, int B, int64_t N_alloc, int64_t N, int H, int H_q, int d,
                    int C, int g, int K_top, int causal, int score_kind, const int32_t *target,
                    double cap, int64_t budget, double *eps, int nthreads);
int orc_bsa(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
            const double *pyr, const int64_t *off, int B, int64_t N, int H, int H_q, int d,
            int C, int g, int K_top, int causal, int32_t *idx, double *score, double *gap,
            int nthreads);
int orc_bsa_scores(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                   const double *pyr, const int64_t *off, int B, int64_t N, int H, int H_q, int d,
                   int C, int g, int K_top, int causal, double *u);
int orc_sparse_attn(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                    const float *K, const float *V, int B, int64_t N_alloc, int64_t N, int H, int H_q,
                    int d, int C, const int32_t *sel, int sel_k, int causal, double *out, double *lse,
                    int nthreads);
int orc_sparse_attn_bwd(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                        const float *K, const float *V, const float *dO, const float *Osaved, int B,
                        int64_t N_alloc, int64_t N, int H, int H_q, int d, int C, const int32_t *sel,
                        int sel_k, int causal, double *dQ, double *dK, double *dV, int nthreads);
int orc_selection_quality(const float *Q, const int64_t *item_b, const int64_t *item_t,
                          int64_t n_items, const float *K, int B, int64_t N_alloc, int64_t N, int H,
                          int H_q, int d, int C, const int32_t *sel, int K_top, double *mass,
                          int32_t *ref, double *recall, double *captured, double *ratio,
                          int nthreads);
double orc_score_kind(const float *q, int64_t b, int h, int l, int64_t i, const float *K,
                      const double *pyr, const int64_t *off, int B, int64_t N_alloc, int64_t N, int H,
                      int d, int C, int g, int kind);

static uint64_t rng = 88172645463325252ull;
static float randn(void)
{
    /* xorshift64 + Box-Muller: synthetic inputs only */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    double u1 = ((rng >> 11) + 1.0) / 9007199254740993.0;
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    double u2 = (rng >> 11) / 9007199254740992.0;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int run(int B, int64_t N, int H, int Hq, int d, int C, int g, int Kt, int causal)
{
    int64_t M[41];
    int L = orc_levels(N, C, g, M);
    if (L < 1) return 1;
    int64_t off[42] = {0}, o = 0;
    for (int l = 1; l <= L; l++) { off[l] = o; o += (int64_t)B * H * M[l] * d; }
    size_t kv = (size_t)B * N * H * d;
    float *K = malloc(kv * sizeof(float)), *V = malloc(kv * sizeof(float));
    for (size_t i = 0; i < kv; i++) { K[i] = randn(); V[i] = randn(); }
    double *pyr = calloc((size_t)o, sizeof(double));
    orc_build_pyramid(K, B, N, N, H, d, C, g, pyr, off);
    int64_t n = N < 40 ? N : 40;
    float *Q = malloc(sizeof(float) * n * Hq * d), *dO = malloc(sizeof(float) * n * Hq * d);
    for (int64_t i = 0; i < n * Hq * d; i++) { Q[i] = randn(); dO[i] = randn(); }
    int64_t *ib = malloc(sizeof(int64_t) * n), *it = malloc(sizeof(int64_t) * n);
    for (int64_t k = 0; k < n; k++) { ib[k] = k % B; it[k] = (k * 7919) % N; }
    int32_t *idx = malloc(sizeof(int32_t) * n * H * Kt), *tr = malloc(sizeof(int32_t) * n * H * (L + 1) * 2);
    double *sc = malloc(sizeof(double) * n * H * Kt), *gap = malloc(sizeof(double) * n * H);
    int bad = 0;
    for (int kind = 2; kind >= 0; kind--)  /* the LSE route last: its output is the target below */
        bad |= orc_route_scored(Q, ib, it, n, K, pyr, off, B, N, N, H, Hq, d, C, g, Kt, causal, kind, idx, sc,
                                gap, tr, 3);
    int32_t *ih = malloc(sizeof(int32_t) * n);
    for (int64_t k = 0; k < n; k++) ih[k] = (int32_t)(k % H);
    int32_t *tg = malloc(sizeof(int32_t) * n * Kt);
    for (int64_t k = 0; k < n; k++) memcpy(tg + k * Kt, idx + (k * H + ih[k]) * Kt, sizeof(int32_t) * Kt);
    double *eps = malloc(sizeof(double) * n);
    bad |= orc_route_reach(Q, ib, it, ih, n, K, pyr, off, B, N, N, H, Hq, d, C, g, Kt, causal, 0, tg, 1e-1,
                           100000, eps, 2);
    for (int64_t k = 0; k < n; k++) bad |= !(eps[k] == 0.0);  /* the route's own output costs 0 */
    bad |= orc_bsa(Q, ib, it, n, pyr, off, B, N, H, Hq, d, C, g, Kt, causal, idx, sc, gap, 2);
    double *u = malloc(sizeof(double) * n * H * M[1]);
    bad |= orc_bsa_scores(Q, ib, it, n, pyr, off, B, N, H, Hq, d, C, g, Kt, causal, u);
    double *out = malloc(sizeof(double) * n * Hq * d), *lse = malloc(sizeof(double) * n * Hq);
    bad |= orc_sparse_attn(Q, ib, it, n, K, V, B, N, N, H, Hq, d, C, idx, Kt, causal, out, lse, 2);
    double *dQ = malloc(sizeof(double) * n * Hq * d);
    double *dK = malloc(sizeof(double) * kv), *dV = malloc(sizeof(double) * kv);
    bad |= orc_sparse_attn_bwd(Q, ib, it, n, K, V, dO, NULL, B, N, N, H, Hq, d, C, idx, Kt, causal, dQ, dK,
                               dV, 2);
    if (causal && Kt >= 3) {
        int32_t *ref = malloc(sizeof(int32_t) * n * H * Kt);
        double *mass = malloc(sizeof(double) * n * H * M[1]), *r1 = malloc(sizeof(double) * n * H),
               *r2 = malloc(sizeof(double) * n * H), *r3 = malloc(sizeof(double) * n * H);
        bad |= orc_selection_quality(Q, ib, it, n, K, B, N, N, H, Hq, d, C, idx, Kt, mass, ref, r1, r2, r3, 2);
        free(ref); free(mass); free(r1); free(r2); free(r3);
    }
    for (int l = 1; l <= L; l++)
        for (int kind = 0; kind < 3; kind++)
            bad |= isnan(orc_score_kind(Q, 0, 0, l, M[l] - 1, K, pyr, off, B, N, N, H, d, C, g, kind));
    free(K); free(V); free(pyr); free(Q); free(dO); free(ib); free(it); free(idx); free(tr); free(sc);
    free(gap); free(ih); free(tg); free(eps); free(u); free(out); free(lse); free(dQ); free(dK); free(dV);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= run(1, 1000, 1, 1, 16, 16, 2, 4, 1);   /* ragged tail, g = 2 */
    bad |= run(2, 777, 2, 4, 8, 16, 4, 6, 1);     /* two sequences, grouped heads, g = 4 */
    bad |= run(1, 512, 2, 8, 8, 8, 3, 5, 0);      /* non-causal, g = 3 */
    bad |= run(1, 70, 1, 2, 4, 16, 2, 3, 1);      /* short: every query keeps all */
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
