/*
 * pisa_oracle.c -- CPU oracle for PISA pyramid Top-K block selection.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow reference that the
 * GPU library is checked against. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may build, load or call it; the product path
 * (hierarchical_top_amd) never does. It shares no code, header, table or
 * helper with the GPU library.
 *
 * Source: "Block Sparse Attention with Log-Linear Complexity" (PISA), arXiv
 * HTML full text. Section, equation and appendix names below refer to that page.
 * The page indexes blocks from 1; this file indexes everything from 0.
 *
 * Arithmetic: every dot product, mean, log-sum-exp and softmax is computed in
 * IEEE double, in the plain order the definitions state (a sum runs over its
 * index in increasing order). Inputs are float32 arrays that hold the exact
 * values the GPU receives (bf16 and fp32 inputs are both exactly
 * representable). No blocking, no fusion, no SIMD intrinsics. Work items are
 * spread over POSIX threads; every item is computed independently, so results
 * do not depend on the thread count.
 *
 * Layouts (all row-major, 0-based):
 *   K, V      [B][N_alloc][H][d]      keys / values, token-major
 *   Q items   [n_items][H_q][d]       one row per routed (sequence, position)
 *   pyramid   level l (1 <= l <= L) at double offset off[l]:
 *             [B][H][M_l][d]
 *   idx/score [n_items][H][K_top]     ascending block ids, -1 padded
 * Query head h' uses KV head h'/G_Q (contiguous grouped-query heads).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAX_LEVELS 40

/* ---------------------------------------------------------------------------
 * Level sizes. Section 3.2, "Fine-to-coarse block aggregation", eq 7, 10, 13:
 *   M_0 = N, M_1 = ceil(N / C), M_{l+1} = ceil(M_l / g) for l >= 1.
 * The coarsest level L is the first level holding a single block: selection
 * starts from the candidate set {first block} at level L (section 3.2,
 * "Coarse-to-fine block selection").
 * Returns L; fills M[0..L]. N must be >= 1.
 * ------------------------------------------------------------------------- */
int orc_levels(int64_t N, int C, int g, int64_t *M)
{
    int L = 1;
    M[0] = N;
    M[1] = (N + C - 1) / C;
    while (M[L] > 1) {
        if (L + 1 > ORC_MAX_LEVELS) return -1;
        M[L + 1] = (M[L] + g - 1) / g;
        L += 1;
    }
    return L;
}

/* Tokens covered by one level-l block: C * g^(l-1) (eq 12, 14). */
static int64_t span_of(int l, int C, int g)
{
    int64_t s = C;
    for (int k = 1; k < l; k++) s *= g;
    return s;
}

/* ---------------------------------------------------------------------------
 * Pyramid build. Section 3.2 eq 15 (with eq 1, 2, 11, 13):
 *   leaf summary  kbar^(1)_i = mean of the keys present in block i,
 *                 i.e. tokens [iC, min(iC + C, N));
 *   level l+1     kbar^(l+1)_i = (1/|Ch_l(i)|) * sum over the existing children
 *                 r in [i g, min(i g + g, M_l)) of kbar^(l)_r.
 * The denominator counts the valid children, so a partial node at the tail is
 * an unweighted mean of its existing children, not a token-weighted mean.
 * Writes levels 1..L of every (b, h). off[l] is the double offset of level l.
 * ------------------------------------------------------------------------- */
void orc_build_pyramid(const float *K, int B, int64_t N_alloc, int64_t N, int H,
                       int d, int C, int g, double *pyr, const int64_t *off)
{
    int64_t M[ORC_MAX_LEVELS + 1];
    int L = orc_levels(N, C, g, M);
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            double *lev1 = pyr + off[1] + ((int64_t)b * H + h) * M[1] * d;
            for (int64_t i = 0; i < M[1]; i++) {
                int64_t lo = i * C, hi = i * C + C < N ? i * C + C : N;
                for (int e = 0; e < d; e++) {
                    double s = 0.0;
                    for (int64_t r = lo; r < hi; r++)
                        s += (double)K[((b * N_alloc + r) * H + h) * (int64_t)d + e];
                    lev1[i * d + e] = s / (double)(hi - lo);
                }
            }
            for (int l = 1; l < L; l++) {
                const double *src = pyr + off[l] + ((int64_t)b * H + h) * M[l] * d;
                double *dst = pyr + off[l + 1] + ((int64_t)b * H + h) * M[l + 1] * d;
                for (int64_t i = 0; i < M[l + 1]; i++) {
                    int64_t lo = i * g, hi = i * g + g < M[l] ? i * g + g : M[l];
                    for (int e = 0; e < d; e++) {
                        double s = 0.0;
                        for (int64_t r = lo; r < hi; r++) s += src[r * d + e];
                        dst[i * d + e] = s / (double)(hi - lo);
                    }
                }
            }
        }
}

/* ---------------------------------------------------------------------------
 * Shared routing problem description.
 * ------------------------------------------------------------------------- */
typedef struct {
    const float *Q;         /* [n_items][H_q][d] */
    const int64_t *item_b;  /* sequence of each item */
    const int64_t *item_t;  /* query position of each item */
    int64_t n_items;
    const float *K;         /* [B][N_alloc][H][d] */
    const float *V;         /* [B][N_alloc][H][d] (attention only) */
    const double *pyr;      /* levels 1..L, layout above */
    const int64_t *off;
    int B, H, H_q, d, C, g, K_top, causal;
    int score_kind;         /* 0 PISA (LSE), 1 PISA-1 (mean), 2 PISA-2 (mean + var / 2) */
    int64_t N, N_alloc;
    int64_t M[ORC_MAX_LEVELS + 1];
    int L;
    /* outputs */
    int32_t *idx;           /* [n_items][H][K_top] */
    double *score;          /* [n_items][H][K_top] */
    double *gap;            /* [n_items][H] (may be NULL) */
    int32_t *trace;         /* [n_items][H][L+1][2]: |A| after filter, #scored (may be NULL) */
    /* attention backward */
    const float *dO;        /* [n_items][H_q][d] gradient of the loss w.r.t. the output */
    const float *Osaved;    /* [n_items][H_q][d] saved forward output, or NULL */
    double *dQ;             /* [n_items][H_q][d] */
    double *dK, *dV;        /* [B][N_alloc][H][d], accumulated */
    const int32_t *sel;     /* attention: selected blocks [n_items][H][K_top] */
    int sel_k;
    double *out;            /* attention: [n_items][H_q][d] */
    double *lse;            /* attention: [n_items][H_q] (may be NULL) */
    /* tie-resolution reachability (orc_route_reach) */
    const int32_t *item_h;  /* KV head of each item */
    const int32_t *target;  /* [n_items][K_top] selection to explain, -1 padded */
    double reach_cap;
    int64_t reach_budget;
    double *reach_eps;      /* [n_items] */
    int nthreads;
} orc_problem;

static double dot_fd(const float *q, const double *k, int d)
{
    double s = 0.0;
    for (int e = 0; e < d; e++) s += (double)q[e] * k[e];
    return s;
}

static double dot_ff(const float *q, const float *k, int d)
{
    double s = 0.0;
    for (int e = 0; e < d; e++) s += (double)q[e] * (double)k[e];
    return s;
}

/* log(sum_j exp(z_j)) over n >= 1 values, in double. */
static double logsumexp(const double *z, int64_t n)
{
    double m = z[0];
    for (int64_t j = 1; j < n; j++) if (z[j] > m) m = z[j];
    double s = 0.0;
    for (int64_t j = 0; j < n; j++) s += exp(z[j] - m);
    return m + log(s);
}

/* Mean of n >= 1 values (section 4.4 eq 33, appendix A.2 eq 43). */
static double mean_of(const double *z, int64_t n)
{
    double s = 0.0;
    for (int64_t j = 0; j < n; j++) s += z[j];
    return s / (double)n;
}

/* Population variance of n >= 1 values about their mean (appendix A.2 eq 44). */
static double var_of(const double *z, int64_t n)
{
    double mu = mean_of(z, n), s = 0.0;
    for (int64_t j = 0; j < n; j++) s += (z[j] - mu) * (z[j] - mu);
    return s / (double)n;
}

/* The block score from the valid logits z[0..n) of one candidate and head:
 * PISA's log-sum-exp (eq 21 / eq 50), or the truncations of its expansion
 * about the mean with log m dropped (section 4.4 eq 33-34, appendix A.2
 * eq 51-52): PISA-1 keeps the mean, PISA-2 the mean plus half the variance. */
static double reduce_logits(int kind, const double *z, int64_t n)
{
    if (kind == 1) return mean_of(z, n);
    if (kind == 2) return mean_of(z, n) + 0.5 * var_of(z, n);
    return logsumexp(z, n);
}

/* ---------------------------------------------------------------------------
 * LSE block score of one candidate for one query head. Section 3.2,
 * "LogSumExp block scoring", eq 21:
 *   s^(l)_{t,i} = log sum_{r in Ch_{l-1}(i)} exp(q_t . kbar^(l-1)_r / sqrt(d)).
 * For l = 1 the children are the raw keys of leaf block i (kbar^(0) = k), so
 * a leaf gets its exact raw-key LSE; for l >= 2 they are the existing level-(l-1)
 * summaries. q points at one query head's d values; h is its KV head.
 * With score_kind 1 or 2 the same logits are reduced by reduce_logits instead.
 * ------------------------------------------------------------------------- */
double orc_lse_score(const orc_problem *P, int64_t b, int h, const float *q, int l,
                     int64_t i)
{
    double z[4096];
    int64_t n = 0;
    double scale = 1.0 / sqrt((double)P->d);
    if (l == 1) {
        int64_t lo = i * P->C, hi = i * P->C + P->C < P->N ? i * P->C + P->C : P->N;
        for (int64_t r = lo; r < hi; r++)
            z[n++] = dot_ff(q, P->K + ((b * P->N_alloc + r) * P->H + h) * (int64_t)P->d,
                            P->d) * scale;
    } else {
        const double *src = P->pyr + P->off[l - 1] + (b * P->H + h) * P->M[l - 1] * P->d;
        int64_t lo = i * P->g, hi = i * P->g + P->g < P->M[l - 1] ? i * P->g + P->g : P->M[l - 1];
        for (int64_t r = lo; r < hi; r++) z[n++] = dot_fd(q, src + r * P->d, P->d) * scale;
    }
    return reduce_logits(P->score_kind, z, n);
}

/* Grouped-query sum, section 3.3 eq 22 and appendix A.3 eq 53: the LSE scores
 * of the G_Q query heads sharing KV head h are added, unnormalised. */
static double group_score(const orc_problem *P, int64_t item, int h, int l, int64_t i)
{
    int G = P->H_q / P->H;
    double u = 0.0;
    for (int j = 0; j < G; j++) {
        const float *q = P->Q + (item * P->H_q + (int64_t)h * G + j) * P->d;
        u += orc_lse_score(P, P->item_b[item], h, q, l, i);
    }
    return u;
}

/* Forced set at level l for query t (appendix B, "Causal masking"): the first,
 * previous and current leaf blocks and their ancestor paths, when distinct
 * and eligible. anc_l(x) = x / g^(l-1) is the level-l ancestor of leaf x.
 * Writes up to 3 distinct node ids; returns the count. */
static int forced_set(const orc_problem *P, int64_t t, int l, int64_t *F)
{
    int64_t c = t / P->C;
    int64_t den = span_of(l, P->C, P->g) / P->C;
    int64_t cand[3];
    int nc = 0, nf = 0;
    cand[nc++] = 0;
    cand[nc++] = c / den;
    if (c >= 1) cand[nc++] = (c - 1) / den;
    for (int k = 0; k < nc; k++) {
        int dup = 0;
        for (int j = 0; j < nf; j++) if (F[j] == cand[k]) dup = 1;
        if (!dup) F[nf++] = cand[k];
    }
    return nf;
}

typedef struct { double u; int64_t i; } scored_t;

/* Select_K ordering (section 3.2 eq 17): higher score first; on equal scores
 * the lower block index wins (the page leaves ties open; this is the fixed
 * tie-break of this implementation). */
static int cmp_scored(const void *a, const void *b)
{
    const scored_t *x = a, *y = b;
    if (x->u > y->u) return -1;
    if (x->u < y->u) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static int contains(const int64_t *s, int n, int64_t v)
{
    for (int k = 0; k < n; k++) if (s[k] == v) return 1;
    return 0;
}

/* Write an ascending, -1 padded selection with its scores. */
static void emit(const orc_problem *P, int64_t item, int h, int64_t *I, double *Iu, int nI)
{
    /* sort (id, score) pairs by id */
    for (int a = 1; a < nI; a++)
        for (int b = a; b > 0 && I[b - 1] > I[b]; b--) {
            int64_t ti = I[b]; I[b] = I[b - 1]; I[b - 1] = ti;
            double tu = Iu[b]; Iu[b] = Iu[b - 1]; Iu[b - 1] = tu;
        }
    int32_t *oi = P->idx + (item * P->H + h) * (int64_t)P->K_top;
    double *os = P->score + (item * P->H + h) * (int64_t)P->K_top;
    for (int k = 0; k < P->K_top; k++) {
        oi[k] = k < nI ? (int32_t)I[k] : -1;
        os[k] = k < nI ? Iu[k] : -INFINITY;
    }
}

/* ---------------------------------------------------------------------------
 * PISA route of one (item, KV head). Section 3.2 eq 16-20, with the forced
 * policy and eligibility rule of appendix B:
 *   A <- {0} at the coarsest level L;
 *   for l = L .. 1:
 *     drop candidates that start after the query (causal);
 *     if |A| <= K_top: keep all of A without scoring;
 *     else: score every non-forced candidate by the grouped LSE (eq 21-22),
 *           keep the forced nodes plus the best K_top - |F| others;
 *     for l > 1: A <- the existing children of the kept nodes (eq 18).
 * The output is the kept leaf set. Scores: the leaf-level grouped score for a
 * leaf kept by ranking, +inf for a leaf kept without a score (forced, or the
 * leaf level held at most K_top candidates). gap = the smallest, over every
 * level that ranked, of (score of the last kept) - (score of the first dropped).
 * ------------------------------------------------------------------------- */
static void route_one(const orc_problem *P, int64_t item, int h)
{
    int64_t t = P->item_t[item];
    int Kt = P->K_top;
    /* |A| <= g * K_top <= 4096 (eq 20), enforced by setup() */
    int64_t *A = malloc(sizeof(int64_t) * 4096);
    int64_t nA = 1;
    int64_t I[4096];
    double Iu[4096];
    int nI = 0;
    scored_t *S = malloc(sizeof(scored_t) * 4096);
    double gap = INFINITY;
    A[0] = 0;
    for (int l = P->L; l >= 1; l--) {
        /* eligibility: a level-l node i covers tokens starting at i * span(l) */
        if (P->causal) {
            int64_t span = span_of(l, P->C, P->g), w = 0;
            for (int64_t k = 0; k < nA; k++) if (A[k] * span <= t) A[w++] = A[k];
            nA = w;
        }
        int64_t F[3];
        int nF = P->causal ? forced_set(P, t, l, F) : 0;
        int nscored = 0;
        if (nA <= Kt) {
            nI = (int)nA;
            for (int64_t k = 0; k < nA; k++) { I[k] = A[k]; Iu[k] = INFINITY; }
        } else {
            int64_t ns = 0;
            for (int64_t k = 0; k < nA; k++) {
                if (contains(F, nF, A[k])) continue;
                S[ns].i = A[k];
                S[ns].u = group_score(P, item, h, l, A[k]);
                ns++;
            }
            nscored = (int)ns;
            qsort(S, (size_t)ns, sizeof(scored_t), cmp_scored);
            int keep = Kt - nF;
            nI = 0;
            for (int k = 0; k < nF; k++) { I[nI] = F[k]; Iu[nI] = INFINITY; nI++; }
            for (int k = 0; k < keep; k++) { I[nI] = S[k].i; Iu[nI] = S[k].u; nI++; }
            if (keep >= 1 && keep < ns) {
                double gp = S[keep - 1].u - S[keep].u;
                if (gp < gap) gap = gp;
            }
        }
        if (P->trace) {
            int32_t *tr = P->trace + ((item * P->H + h) * (int64_t)(P->L + 1) + l) * 2;
            tr[0] = (int32_t)nA;
            tr[1] = nscored;
        }
        if (l > 1) {
            nA = 0;
            for (int k = 0; k < nI; k++) {
                int64_t lo = I[k] * P->g;
                int64_t hi = lo + P->g < P->M[l - 1] ? lo + P->g : P->M[l - 1];
                for (int64_t r = lo; r < hi; r++) A[nA++] = r;
            }
            qsort(A, (size_t)nA, sizeof(int64_t), cmp_i64);
        }
    }
    emit(P, item, h, I, Iu, nI);
    if (P->gap) P->gap[item * P->H + h] = gap;
    free(A);
    free(S);
}

/* ---------------------------------------------------------------------------
 * Tie-resolution reachability of a given selection (checker for near ties).
 *
 * Select_K (section 3.2 eq 17) is exact only up to the precision of the
 * scores: two implementations whose scores differ by rounding may resolve a
 * near tie differently at some level and then descend into another subtree.
 * This function decides whether a selection T of one (item, KV head) is the
 * outcome of such a resolution. It walks the same levels as route_one, but at
 * every level that ranks it tries each kept set S of the non-forced candidates
 * R with |S| = K_top - |F| whose swap cost
 *     cost(S) = max(0, max over R \ S of u - min over S of u)
 * is at most cap (cost 0 is the ordinary Top-K; a positive cost means a
 * candidate scoring up to that much above a kept one was dropped). A path's
 * cost is the largest cost of its levels. The result is the smallest path
 * cost among the paths whose kept leaf set equals T: 0 when T is the route's
 * own output, +inf when no path within cap reaches T, NaN when the search
 * exceeded budget visited kept sets before finding any path (undecided; a
 * path found before that bounds the smallest cost from above).
 * Only kept sets that contain the level-l ancestors of every leaf of T can
 * lead to T (a leaf is reached only through its ancestors), which keeps the
 * search small; and since |S| is fixed, an S of cost <= cap holds every
 * candidate scoring above the (K_top - |F|)-th score plus cap and none below
 * the next score minus cap, so only the candidates between those bounds are
 * enumerated.
 * ------------------------------------------------------------------------- */
typedef struct {
    const orc_problem *P;
    int64_t item, t;
    int h;
    int64_t tgt[4096];
    int ntgt;
    double cap, best;
    int64_t budget, visits;
    int overflow;
} reach_ctx;

static void reach_level(reach_ctx *R, int l, const int64_t *Ain, int64_t nAin, double cost);

/* Continue from kept set I (nI ids) of level l with path cost `cost`. */
static void reach_next(reach_ctx *R, int l, int64_t *I, int64_t nI, double cost)
{
    const orc_problem *P = R->P;
    if (l == 1) {
        qsort(I, (size_t)nI, sizeof(int64_t), cmp_i64);
        if (nI != R->ntgt) return;
        for (int64_t k = 0; k < nI; k++) if (I[k] != R->tgt[k]) return;
        if (cost < R->best) R->best = cost;
        return;
    }
    int64_t *A = malloc(sizeof(int64_t) * (size_t)(nI * P->g > 0 ? nI * P->g : 1));
    int64_t nA = 0;
    for (int64_t k = 0; k < nI; k++) {
        int64_t lo = I[k] * P->g, hi = lo + P->g < P->M[l - 1] ? lo + P->g : P->M[l - 1];
        for (int64_t r = lo; r < hi; r++) A[nA++] = r;
    }
    qsort(A, (size_t)nA, sizeof(int64_t), cmp_i64);
    reach_level(R, l - 1, A, nA, cost);
    free(A);
}

static void reach_level(reach_ctx *R, int l, const int64_t *Ain, int64_t nAin, double cost)
{
    const orc_problem *P = R->P;
    if (R->overflow || cost >= R->best) return;
    int64_t span = span_of(l, P->C, P->g), den = span / P->C;
    int64_t *A = malloc(sizeof(int64_t) * (size_t)(nAin > 0 ? nAin : 1));
    int64_t *I = malloc(sizeof(int64_t) * (size_t)(nAin + 3));
    scored_t *S = malloc(sizeof(scored_t) * (size_t)(nAin > 0 ? nAin : 1));
    char *st = malloc((size_t)(nAin > 0 ? nAin : 1));      /* 0 out, 1 sure in, 2 pool, 3 required */
    int64_t *pool = malloc(sizeof(int64_t) * (size_t)(nAin > 0 ? nAin : 1));
    int64_t *cmb = malloc(sizeof(int64_t) * (size_t)(nAin > 0 ? nAin : 1));
    int64_t nA = 0;
    for (int64_t k = 0; k < nAin; k++)
        if (!P->causal || Ain[k] * span <= R->t) A[nA++] = Ain[k];
    /* every leaf of T must still be reachable through a candidate of this level */
    for (int j = 0; j < R->ntgt; j++)
        if (!contains(A, (int)nA, R->tgt[j] / den)) goto done;
    if (nA <= P->K_top) {
        memcpy(I, A, sizeof(int64_t) * (size_t)nA);
        reach_next(R, l, I, nA, cost);
        goto done;
    }
    {
        int64_t F[3];
        int nF = P->causal ? forced_set(P, R->t, l, F) : 0;
        int64_t ns = 0;
        for (int64_t k = 0; k < nA; k++) {
            if (contains(F, nF, A[k])) continue;
            S[ns].i = A[k];
            S[ns].u = group_score(P, R->item, R->h, l, A[k]);
            ns++;
        }
        qsort(S, (size_t)ns, sizeof(scored_t), cmp_scored);
        int64_t keep = P->K_top - nF;
        double hi = keep >= 1 ? S[keep - 1].u : INFINITY;
        double lo = keep < ns ? S[keep].u : -INFINITY;
        int64_t nsure = 0, npool = 0, nreq = 0;
        for (int64_t k = 0; k < ns; k++) {
            int req = 0;
            for (int j = 0; j < R->ntgt; j++) if (R->tgt[j] / den == S[k].i) req = 1;
            if (S[k].u > hi + R->cap) st[k] = 1;
            else if (S[k].u < lo - R->cap) st[k] = 0;
            else st[k] = 2;
            if (req && st[k] == 0) goto done;        /* a needed ancestor cannot be kept */
            if (req && st[k] == 2) st[k] = 3;
            if (st[k] == 1) nsure++;
            if (st[k] == 3) nreq++;
            if (st[k] == 2) pool[npool++] = k;
        }
        int64_t m = keep - nsure - nreq;              /* free picks from the pool */
        if (m < 0 || m > npool) goto done;
        for (int64_t k = 0; k < m; k++) cmb[k] = k;
        for (;;) {
            if (++R->visits > R->budget) { R->overflow = 1; break; }
            /* kept set: sure + required + pool[cmb[0..m)] */
            char *in = st;  /* reuse: mark chosen pool entries as 4 temporarily */
            for (int64_t k = 0; k < m; k++) in[pool[cmb[k]]] = 4;
            double mn = INFINITY, mx = -INFINITY;
            int64_t nI = 0;
            for (int k = 0; k < nF; k++) I[nI++] = F[k];
            for (int64_t k = 0; k < ns; k++) {
                if (in[k] == 1 || in[k] == 3 || in[k] == 4) {
                    I[nI++] = S[k].i;
                    if (S[k].u < mn) mn = S[k].u;
                } else if (S[k].u > mx) {
                    mx = S[k].u;
                }
            }
            for (int64_t k = 0; k < m; k++) in[pool[cmb[k]]] = 2;
            double cl = mx - mn > 0.0 ? mx - mn : 0.0;
            double nc = cl > cost ? cl : cost;
            if (cl <= R->cap && nc < R->best) reach_next(R, l, I, nI, nc);
            if (R->overflow || R->best <= cost) break;  /* cannot improve further */
            /* next combination of m out of npool (lexicographic) */
            int64_t k = m - 1;
            while (k >= 0 && cmb[k] == npool - m + k) k--;
            if (k < 0) break;
            cmb[k]++;
            for (int64_t j = k + 1; j < m; j++) cmb[j] = cmb[j - 1] + 1;
        }
    }
done:
    free(A); free(I); free(S); free(st); free(pool); free(cmb);
}

static void reach_one(const orc_problem *P, int64_t item)
{
    reach_ctx *R = malloc(sizeof(reach_ctx));
    R->P = P;
    R->item = item;
    R->t = P->item_t[item];
    R->h = P->item_h[item];
    R->ntgt = 0;
    const int32_t *T = P->target + item * (int64_t)P->K_top;
    for (int k = 0; k < P->K_top; k++) if (T[k] >= 0) R->tgt[R->ntgt++] = T[k];
    qsort(R->tgt, (size_t)R->ntgt, sizeof(int64_t), cmp_i64);
    R->cap = P->reach_cap;
    R->best = INFINITY;
    R->budget = P->reach_budget;
    R->visits = 0;
    R->overflow = 0;
    int64_t root = 0;
    reach_level(R, P->L, &root, 1, 0.0);
    /* on overflow a path already found still bounds the smallest cost from above */
    P->reach_eps[item] = (R->overflow && isinf(R->best)) ? NAN : R->best;
    free(R);
}

/* ---------------------------------------------------------------------------
 * Exhaustive single-level selector in the style of BSA (section 3.1 eq 2-5),
 * with the grouped-query rule the page describes for its BSA baseline
 * (section 4.1 and appendix C: scores are normalised within each query head
 * before they are summed over the heads of the group):
 *   z_{h',i} = q_{t,h'} . kbar_i / sqrt(d) over the scored leaves S,
 *   p_{h',i} = softmax over i in S of z_{h',i},   u_i = sum_{h'} p_{h',i}.
 * S = the eligible leaves (start <= t when causal) minus the forced set; the
 * forced leaves are kept; if at most K_top leaves are eligible all are kept.
 * kbar_i is the level-1 summary of the pyramid (mean pooling, eq 2).
 * ------------------------------------------------------------------------- */
/* u_i = sum over the group's heads of the per-head softmax of z_{h',i} over the
 * scored leaves S[0..ns) (ids set by the caller; u written into S[k].u). */
static void bsa_group_probs(const orc_problem *P, int64_t item, int h, scored_t *S, int64_t ns)
{
    int64_t b = P->item_b[item];
    int G = P->H_q / P->H;
    double *z = malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
    const double *lev1 = P->pyr + P->off[1] + (b * P->H + h) * P->M[1] * P->d;
    double scale = 1.0 / sqrt((double)P->d);
    for (int64_t k = 0; k < ns; k++) S[k].u = 0.0;
    for (int j = 0; j < G; j++) {
        const float *q = P->Q + (item * P->H_q + (int64_t)h * G + j) * P->d;
        for (int64_t k = 0; k < ns; k++) z[k] = dot_fd(q, lev1 + S[k].i * P->d, P->d) * scale;
        double lz = logsumexp(z, ns);
        for (int64_t k = 0; k < ns; k++) S[k].u += exp(z[k] - lz);
    }
    free(z);
}

/* The eligible leaf count of query t (all M_1 leaves when not causal) and the
 * scored set: eligible minus forced; returns ns. */
static int64_t bsa_scored_set(const orc_problem *P, int64_t t, scored_t *S, int64_t *E_out,
                              int64_t *F, int *nF_out)
{
    int64_t E = P->causal ? t / P->C + 1 : P->M[1];
    if (E > P->M[1]) E = P->M[1];
    int nF = P->causal ? forced_set(P, t, 1, F) : 0;
    int64_t ns = 0;
    for (int64_t i = 0; i < E; i++) {
        if (contains(F, nF, i)) continue;
        S[ns].i = i;
        S[ns].u = 0.0;
        ns++;
    }
    *E_out = E;
    *nF_out = nF;
    return ns;
}

static void bsa_one(const orc_problem *P, int64_t item, int h)
{
    int64_t t = P->item_t[item];
    int Kt = P->K_top;
    int64_t I[4096];
    double Iu[4096];
    int nI = 0;
    double gap = INFINITY;
    int64_t E, F[3];
    int nF;
    scored_t *S = malloc(sizeof(scored_t) * (size_t)P->M[1]);
    int64_t ns = bsa_scored_set(P, t, S, &E, F, &nF);
    if (E <= Kt) {
        for (int64_t i = 0; i < E; i++) { I[nI] = i; Iu[nI] = INFINITY; nI++; }
    } else {
        bsa_group_probs(P, item, h, S, ns);
        qsort(S, (size_t)ns, sizeof(scored_t), cmp_scored);
        int keep = Kt - nF;
        for (int k = 0; k < nF; k++) { I[nI] = F[k]; Iu[nI] = INFINITY; nI++; }
        for (int k = 0; k < keep; k++) { I[nI] = S[k].i; Iu[nI] = S[k].u; nI++; }
        if (keep >= 1 && keep < ns) gap = S[keep - 1].u - S[keep].u;
    }
    free(S);
    emit(P, item, h, I, Iu, nI);
    if (P->gap) P->gap[item * P->H + h] = gap;
}

/* ---------------------------------------------------------------------------
 * Block-sparse attention of one (item, query head). Section 3.1 eq 6:
 *   o_t = sum_{j in T_t} exp(q_t . k_j / sqrt(d)) v_j / sum_{j in T_t} exp(...),
 * T_t = the tokens of the selected blocks of the query's KV head; under causal
 * masking the tokens after the query are left out (appendix B: the attention
 * kernel masks future tokens inside selected blocks). A query with no token
 * (an empty selection) gets a zero output and lse = -inf.
 * ------------------------------------------------------------------------- */
static void attn_one(const orc_problem *P, int64_t item, int hq)
{
    int G = P->H_q / P->H;
    int h = hq / G;
    int64_t t = P->item_t[item], b = P->item_b[item];
    const float *q = P->Q + (item * P->H_q + hq) * P->d;
    const int32_t *sel = P->sel + (item * P->H + h) * (int64_t)P->sel_k;
    double scale = 1.0 / sqrt((double)P->d);
    int64_t cap = (int64_t)P->sel_k * P->C;
    double *z = malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    int64_t *tok = malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    int64_t n = 0;
    for (int k = 0; k < P->sel_k; k++) {
        int64_t i = sel[k];
        if (i < 0) continue;
        int64_t lo = i * P->C, hi = i * P->C + P->C < P->N ? i * P->C + P->C : P->N;
        for (int64_t j = lo; j < hi; j++) {
            if (P->causal && j > t) continue;
            tok[n] = j;
            z[n] = dot_ff(q, P->K + ((b * P->N_alloc + j) * P->H + h) * (int64_t)P->d, P->d) * scale;
            n++;
        }
    }
    double *o = P->out + (item * P->H_q + hq) * P->d;
    for (int e = 0; e < P->d; e++) o[e] = 0.0;
    if (n == 0) {
        if (P->lse) P->lse[item * P->H_q + hq] = -INFINITY;
    } else {
        double lz = logsumexp(z, n);
        for (int64_t k = 0; k < n; k++) {
            double p = exp(z[k] - lz);
            const float *v = P->V + ((b * P->N_alloc + tok[k]) * P->H + h) * (int64_t)P->d;
            for (int e = 0; e < P->d; e++) o[e] += p * (double)v[e];
        }
        if (P->lse) P->lse[item * P->H_q + hq] = lz;
    }
    free(z);
    free(tok);
}

/* ---------------------------------------------------------------------------
 * Backward of block-sparse attention (section 3.1 eq 6; section 3.3: during
 * training the gradients flow through attention on the selected entries only,
 * the selection itself is not differentiated). For one query head with token
 * set T (as in attn_one), z_j = q . k_j / sqrt(d), p = softmax(z) over T,
 * o = sum_j p_j v_j and an upstream gradient dO of o:
 *   dv_j += p_j dO                          (o is linear in v)
 *   dp_j  = dO . v_j
 *   dz_j  = p_j (dp_j - sum_{k in T} p_k dp_k)   (Jacobian of the softmax)
 *   dq   += sum_j dz_j k_j / sqrt(d)
 *   dk_j += dz_j q / sqrt(d)
 * Since sum_k p_k dp_k = dO . o, a backward that is handed the saved forward
 * output O uses dO . O in its place (Osaved non-NULL): the two agree exactly
 * when O is the exact output, and differ by dO . (O - o) when O was rounded.
 * Every (item, query head) of KV head h of sequence b adds into the same dK,
 * dV rows, so one task owns one (b, h) and visits its items in increasing
 * order and the G_Q query heads in increasing order.
 * ------------------------------------------------------------------------- */
static void attn_bwd_one(const orc_problem *P, int64_t item, int hq)
{
    int G = P->H_q / P->H;
    int h = hq / G;
    int64_t t = P->item_t[item], b = P->item_b[item];
    const float *q = P->Q + (item * P->H_q + hq) * P->d;
    const float *dO = P->dO + (item * P->H_q + hq) * P->d;
    const int32_t *sel = P->sel + (item * P->H + h) * (int64_t)P->sel_k;
    double scale = 1.0 / sqrt((double)P->d);
    int64_t cap = (int64_t)P->sel_k * P->C;
    double *z = malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    double *dp = malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    int64_t *tok = malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    int64_t n = 0;
    for (int k = 0; k < P->sel_k; k++) {
        int64_t i = sel[k];
        if (i < 0) continue;
        int64_t lo = i * P->C, hi = i * P->C + P->C < P->N ? i * P->C + P->C : P->N;
        for (int64_t j = lo; j < hi; j++) {
            if (P->causal && t < j) continue;  /* future token */
            tok[n] = j;
            z[n] = dot_ff(q, P->K + ((b * P->N_alloc + j) * P->H + h) * (int64_t)P->d, P->d) * scale;
            n++;
        }
    }
    double *dq = P->dQ + (item * P->H_q + hq) * P->d;
    for (int e = 0; e < P->d; e++) dq[e] = 0.0;
    if (n > 0) {
        double lz = logsumexp(z, n);
        double pdp = 0.0;  /* sum_k p_k dp_k */
        for (int64_t k = 0; k < n; k++) {
            const float *v = P->V + ((b * P->N_alloc + tok[k]) * P->H + h) * (int64_t)P->d;
            dp[k] = dot_ff(dO, v, P->d);
            pdp += exp(z[k] - lz) * dp[k];
        }
        if (P->Osaved) pdp = dot_ff(dO, P->Osaved + (item * P->H_q + hq) * P->d, P->d);
        for (int64_t k = 0; k < n; k++) {
            double p = exp(z[k] - lz);
            double dz = p * (dp[k] - pdp);
            int64_t row = ((b * P->N_alloc + tok[k]) * P->H + h) * (int64_t)P->d;
            const float *kk = P->K + row;
            for (int e = 0; e < P->d; e++) {
                P->dV[row + e] += p * (double)dO[e];
                P->dK[row + e] += dz * scale * (double)q[e];
                dq[e] += dz * scale * (double)kk[e];
            }
        }
    }
    free(z);
    free(dp);
    free(tok);
}

static void attn_bwd_group(const orc_problem *P, int64_t b, int h)
{
    int G = P->H_q / P->H;
    for (int64_t item = 0; item < P->n_items; item++) {
        if (P->item_b[item] != b) continue;
        for (int hq = h * G; hq < h * G + G; hq++) attn_bwd_one(P, item, hq);
    }
}

/* ---------------------------------------------------------------------------
 * Thread pool: task k of n is handled by thread k % nthreads.
 * ------------------------------------------------------------------------- */
typedef struct {
    const orc_problem *P;
    int which;   /* 0 route, 1 bsa, 2 attention, 3 attention backward, 4 reachability */
    int tid;
} worker_arg;

static void *worker(void *p)
{
    worker_arg *w = p;
    const orc_problem *P = w->P;
    if (w->which == 3) {  /* attention backward: one task per (sequence, KV head) */
        for (int64_t k = w->tid; k < (int64_t)P->B * P->H; k += P->nthreads)
            attn_bwd_group(P, k / P->H, (int)(k % P->H));
        return NULL;
    }
    if (w->which == 4) {  /* reachability: one task per item (its KV head is item_h) */
        for (int64_t k = w->tid; k < P->n_items; k += P->nthreads) reach_one(P, k);
        return NULL;
    }
    int per = w->which == 2 ? P->H_q : P->H;
    int64_t n = P->n_items * per;
    for (int64_t k = w->tid; k < n; k += P->nthreads) {
        int64_t item = k / per;
        int h = (int)(k % per);
        if (w->which == 0) route_one(P, item, h);
        else if (w->which == 1) bsa_one(P, item, h);
        else attn_one(P, item, h);
    }
    return NULL;
}

static void run_pool(const orc_problem *P, int which)
{
    int nt = P->nthreads < 1 ? 1 : P->nthreads;
    pthread_t th[256];
    worker_arg wa[256];
    if (nt > 256) nt = 256;
    orc_problem Pc = *P;
    Pc.nthreads = nt;
    for (int k = 0; k < nt; k++) {
        wa[k].P = &Pc; wa[k].which = which; wa[k].tid = k;
        pthread_create(&th[k], NULL, worker, &wa[k]);
    }
    for (int k = 0; k < nt; k++) pthread_join(th[k], NULL);
}

static int setup(orc_problem *P, const float *Q, const int64_t *item_b, const int64_t *item_t,
                 int64_t n_items, const float *K, const double *pyr, const int64_t *off,
                 int B, int64_t N_alloc, int64_t N, int H, int H_q, int d, int C, int g,
                 int K_top, int causal, int nthreads)
{
    memset(P, 0, sizeof(*P));
    if (N < 1 || C < 1 || g < 2 || H < 1 || H_q % H != 0 || d < 1 || K_top < 1) return -1;
    if (C > 4096 || g > 4096) return -1;
    P->Q = Q; P->item_b = item_b; P->item_t = item_t; P->n_items = n_items;
    P->K = K; P->pyr = pyr; P->off = off;
    P->B = B; P->H = H; P->H_q = H_q; P->d = d; P->C = C; P->g = g;
    P->K_top = K_top; P->causal = causal; P->N = N; P->N_alloc = N_alloc;
    P->nthreads = nthreads;
    P->L = orc_levels(N, C, g, P->M);
    if (P->L < 1) return -1;
    if (causal && K_top < 3) return -1;
    if ((int64_t)K_top * g > 4096 || (int64_t)K_top * C > 4096 * 4) return -1;
    for (int64_t k = 0; k < n_items; k++)
        if (item_b[k] < 0 || item_b[k] >= B || item_t[k] < 0 || item_t[k] >= N) return -1;
    return 0;
}

/* Route n_items queries for every KV head with block score score_kind (0 PISA,
 * 1 PISA-1, 2 PISA-2; the hierarchy, forced set and expansion are the same for
 * all three, section 4.4). Returns 0, or -1 on bad input. */
int orc_route_scored(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                     const float *K, const double *pyr, const int64_t *off, int B, int64_t N_alloc,
                     int64_t N, int H, int H_q, int d, int C, int g, int K_top, int causal,
                     int score_kind, int32_t *idx, double *score, double *gap, int32_t *trace,
                     int nthreads)
{
    orc_problem P;
    if (score_kind < 0 || score_kind > 2) return -1;
    if (setup(&P, Q, item_b, item_t, n_items, K, pyr, off, B, N_alloc, N, H, H_q, d, C, g,
              K_top, causal, nthreads)) return -1;
    P.score_kind = score_kind;
    P.idx = idx; P.score = score; P.gap = gap; P.trace = trace;
    run_pool(&P, 0);
    return 0;
}

/* Route n_items queries for every KV head (PISA). Returns 0, or -1 on bad input. */
int orc_route(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
              const float *K, const double *pyr, const int64_t *off, int B, int64_t N_alloc,
              int64_t N, int H, int H_q, int d, int C, int g, int K_top, int causal,
              int32_t *idx, double *score, double *gap, int32_t *trace, int nthreads)
{
    return orc_route_scored(Q, item_b, item_t, n_items, K, pyr, off, B, N_alloc, N, H, H_q, d, C,
                            g, K_top, causal, 0, idx, score, gap, trace, nthreads);
}

/* Smallest tie-resolution cost (see reach_one) at which the route of item k
 * for KV head item_h[k] can end in the selection target [n_items][K_top]
 * (ascending or not, -1 padded), searching kept sets of cost <= cap and at
 * most budget of them per item. eps [n_items]. Returns 0 or -1. */
int orc_route_reach(const float *Q, const int64_t *item_b, const int64_t *item_t,
                    const int32_t *item_h, int64_t n_items, const float *K, const double *pyr,
                    const int64_t *off, int B, int64_t N_alloc, int64_t N, int H, int H_q, int d,
                    int C, int g, int K_top, int causal, int score_kind, const int32_t *target,
                    double cap, int64_t budget, double *eps, int nthreads)
{
    orc_problem P;
    if (score_kind < 0 || score_kind > 2 || !(cap >= 0.0) || budget < 1) return -1;
    if (setup(&P, Q, item_b, item_t, n_items, K, pyr, off, B, N_alloc, N, H, H_q, d, C, g,
              K_top, causal, nthreads)) return -1;
    for (int64_t k = 0; k < n_items; k++)
        if (item_h[k] < 0 || item_h[k] >= H) return -1;
    P.score_kind = score_kind;
    P.item_h = item_h; P.target = target; P.reach_cap = cap; P.reach_budget = budget;
    P.reach_eps = eps;
    run_pool(&P, 4);
    return 0;
}

/* Exhaustive BSA-style selection for n_items queries. Returns 0 or -1. */
int orc_bsa(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
            const double *pyr, const int64_t *off, int B, int64_t N, int H, int H_q, int d,
            int C, int g, int K_top, int causal, int32_t *idx, double *score, double *gap,
            int nthreads)
{
    orc_problem P;
    if (setup(&P, Q, item_b, item_t, n_items, NULL, pyr, off, B, N, N, H, H_q, d, C, g,
              K_top, causal, nthreads)) return -1;
    P.idx = idx; P.score = score; P.gap = gap;
    run_pool(&P, 1);
    return 0;
}

/* Every leaf's BSA score for n_items queries and every KV head:
 * u [n_items][H][M_1] holds u_i of eq 3-5 (per-head softmax, summed over the
 * group) for a scored leaf, +inf for a leaf kept without a score (forced, or
 * every eligible leaf when at most K_top are eligible) and -inf for a leaf
 * after the query. Exposed so tests can check the normalisation itself.
 * Returns 0 or -1. */
int orc_bsa_scores(const float *Q, const int64_t *item_b, const int64_t *item_t, int64_t n_items,
                   const double *pyr, const int64_t *off, int B, int64_t N, int H, int H_q, int d,
                   int C, int g, int K_top, int causal, double *u)
{
    orc_problem P;
    if (setup(&P, Q, item_b, item_t, n_items, NULL, pyr, off, B, N, N, H, H_q, d, C, g,
              K_top, causal, 1)) return -1;
    scored_t *S = malloc(sizeof(scored_t) * (size_t)P.M[1]);
    for (int64_t item = 0; item < n_items; item++)
        for (int h = 0; h < H; h++) {
            double *o = u + (item * H + h) * P.M[1];
            int64_t E, F[3];
            int nF;
            int64_t ns = bsa_scored_set(&P, item_t[item], S, &E, F, &nF);
            for (int64_t i = 0; i < P.M[1]; i++) o[i] = i < E ? INFINITY : -INFINITY;
            if (E <= K_top) continue;
            bsa_group_probs(&P, item, h, S, ns);
            for (int64_t k = 0; k < ns; k++) o[S[k].i] = S[k].u;
        }
    free(S);
    return 0;
}

/* Block-sparse attention for n_items queries over the given selections
 * sel [n_items][H][sel_k]. out [n_items][H_q][d], lse [n_items][H_q] (nullable). */
int orc_sparse_attn(const float *Q, const int64_t *item_b, const int64_t *item_t,
                    int64_t n_items, const float *K, const float *V, int B, int64_t N_alloc,
                    int64_t N, int H, int H_q, int d, int C, const int32_t *sel, int sel_k,
                    int causal, double *out, double *lse, int nthreads)
{
    orc_problem P;
    if (setup(&P, Q, item_b, item_t, n_items, K, NULL, NULL, B, N_alloc, N, H, H_q, d, C, 2,
              3, 0, nthreads)) return -1;
    P.V = V; P.sel = sel; P.sel_k = sel_k; P.causal = causal; P.out = out; P.lse = lse;
    run_pool(&P, 2);
    return 0;
}

/* Backward of block-sparse attention for n_items queries over sel [n_items][H][sel_k],
 * given dO [n_items][H_q][d] and optionally the saved forward output O (same
 * layout, NULL: none). Writes dQ [n_items][H_q][d]; dK and dV
 * [B][N_alloc][H][d] are set to zero and then accumulate every item's part. */
int orc_sparse_attn_bwd(const float *Q, const int64_t *item_b, const int64_t *item_t,
                        int64_t n_items, const float *K, const float *V, const float *dO,
                        const float *Osaved, int B, int64_t N_alloc, int64_t N, int H, int H_q,
                        int d, int C, const int32_t *sel, int sel_k, int causal, double *dQ,
                        double *dK, double *dV, int nthreads)
{
    orc_problem P;
    if (setup(&P, Q, item_b, item_t, n_items, K, NULL, NULL, B, N_alloc, N, H, H_q, d, C, 2,
              3, 0, nthreads)) return -1;
    for (int64_t k = 0; k < n_items; k++)
        if (item_b[k] < 0 || item_b[k] >= B) return -1;
    P.V = V; P.sel = sel; P.sel_k = sel_k; P.causal = causal;
    P.dO = dO; P.Osaved = Osaved; P.dQ = dQ; P.dK = dK; P.dV = dV;
    size_t kv = (size_t)B * (size_t)N_alloc * (size_t)H * (size_t)d;
    memset(dK, 0, kv * sizeof(double));
    memset(dV, 0, kv * sizeof(double));
    run_pool(&P, 3);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Block-selection quality against full attention (section 4.4 eq 35-36,
 * appendix D.2 eq 55-57), causal. For query position i of sequence b, KV head h
 * and its query heads h', over the eligible leaf blocks E_i = {0..c}, c = i / C:
 *   a_{h'}(B) = log sum_{t in B, t <= i} exp(q_{i,h'} . k_{t,h} / sqrt(d))   (eq 55)
 *   P(B) = (1/G) sum_{h'} exp(a_{h'}(B)) / sum_{B' in E_i} exp(a_{h'}(B'))  (eq 56)
 * The reference set keeps the forced blocks (first, previous, current) and
 * fills the remaining K_top - |F| slots with the other eligible blocks of
 * highest P (ties to the lower index); all of E_i when |E_i| <= K_top. For the
 * selector's set I (sel, -1 entries ignored):
 *   Recall@K = |I cap I_full| / K_top                                     (eq 35)
 *   Captured = sum_{B in I} P(B)                                           (eq 57)
 *   MassRatio = Captured / sum_{B in I_full} P(B)                          (eq 36)
 * ------------------------------------------------------------------------- */
typedef struct {
    const float *Q, *K;
    const int64_t *item_b, *item_t;
    const int32_t *sel;
    int64_t n_items, N, N_alloc;
    int H, H_q, d, C, K_top;
    double *mass;            /* [n_items][H][M_1] or NULL */
    int32_t *ref;            /* [n_items][H][K_top] */
    double *recall, *captured, *ratio;  /* [n_items][H] */
    int nthreads;
} orc_quality;

static void quality_one(const orc_quality *P, int64_t item, int h)
{
    int G = P->H_q / P->H;
    int64_t i = P->item_t[item], b = P->item_b[item];
    int64_t c = i / P->C, nE = c + 1, M1 = (P->N + P->C - 1) / P->C;
    double scale = 1.0 / sqrt((double)P->d);
    double *Pm = calloc((size_t)nE, sizeof(double));
    double *a = malloc(sizeof(double) * (size_t)nE);
    double *z = malloc(sizeof(double) * (size_t)P->C);
    for (int g2 = 0; g2 < G; g2++) {
        const float *q = P->Q + (item * P->H_q + h * G + g2) * P->d;
        for (int64_t B = 0; B < nE; B++) {
            int64_t lo = B * P->C, hi = B * P->C + P->C;
            if (hi > i + 1) hi = i + 1;
            int64_t n = 0;
            for (int64_t t = lo; t < hi; t++)
                z[n++] = dot_ff(q, P->K + ((b * P->N_alloc + t) * P->H + h) * (int64_t)P->d, P->d) * scale;
            a[B] = logsumexp(z, n);
        }
        double la = logsumexp(a, nE);
        for (int64_t B = 0; B < nE; B++) Pm[B] += exp(a[B] - la) / (double)G;
    }
    int Kt = P->K_top;
    int32_t *ref = P->ref + (item * P->H + h) * (int64_t)Kt;
    int nr = 0;
    if (nE <= Kt) {
        for (int64_t B = 0; B < nE; B++) ref[nr++] = (int32_t)B;
    } else {
        char *in = calloc((size_t)nE, 1);
        in[0] = 1; in[c] = 1; in[c - 1] = 1;  /* nE > K_top >= 3: c >= 3 */
        int nF = 3;
        for (int k = 0; k < Kt - nF; k++) {
            int64_t best = -1;
            for (int64_t B = 0; B < nE; B++)
                if (!in[B] && (best < 0 || Pm[B] > Pm[best])) best = B;
            in[best] = 1;
        }
        for (int64_t B = 0; B < nE; B++)
            if (in[B]) ref[nr++] = (int32_t)B;
        free(in);
    }
    for (int k = nr; k < Kt; k++) ref[k] = -1;
    const int32_t *s = P->sel + (item * P->H + h) * (int64_t)Kt;
    double cap = 0.0, cap_ref = 0.0;
    int hit = 0;
    for (int k = 0; k < Kt; k++) {
        if (s[k] >= 0 && s[k] < nE) {
            cap += Pm[s[k]];
            for (int r = 0; r < nr; r++) hit += ref[r] == s[k];
        }
    }
    for (int r = 0; r < nr; r++) cap_ref += Pm[ref[r]];
    int64_t o = item * P->H + h;
    P->recall[o] = (double)hit / (double)Kt;
    P->captured[o] = cap;
    P->ratio[o] = cap / cap_ref;
    if (P->mass) {
        double *m = P->mass + o * M1;
        for (int64_t B = 0; B < M1; B++) m[B] = B < nE ? Pm[B] : 0.0;
    }
    free(Pm);
    free(a);
    free(z);
}

typedef struct { const orc_quality *P; int tid; } quality_arg;

static void *quality_worker(void *p)
{
    quality_arg *w = p;
    const orc_quality *P = w->P;
    for (int64_t k = w->tid; k < P->n_items * P->H; k += P->nthreads)
        quality_one(P, k / P->H, (int)(k % P->H));
    return NULL;
}

/* Selection quality of sel [n_items][H][K_top] for causal queries at positions
 * item_t of sequences item_b (K_top >= 3). Returns 0, or -1 on bad input. */
int orc_selection_quality(const float *Q, const int64_t *item_b, const int64_t *item_t,
                          int64_t n_items, const float *K, int B, int64_t N_alloc, int64_t N,
                          int H, int H_q, int d, int C, const int32_t *sel, int K_top,
                          double *mass, int32_t *ref, double *recall, double *captured,
                          double *ratio, int nthreads)
{
    if (B < 1 || N < 1 || N > N_alloc || H < 1 || H_q < H || H_q % H || d < 1 || C < 1 || K_top < 3)
        return -1;
    for (int64_t k = 0; k < n_items; k++)
        if (item_b[k] < 0 || item_b[k] >= B || item_t[k] < 0 || item_t[k] >= N) return -1;
    orc_quality P = {Q, K, item_b, item_t, sel, n_items, N, N_alloc, H, H_q, d, C, K_top,
                     mass, ref, recall, captured, ratio, nthreads < 1 ? 1 : nthreads};
    if (P.nthreads > 256) P.nthreads = 256;
    pthread_t th[256];
    quality_arg wa[256];
    for (int k = 0; k < P.nthreads; k++) {
        wa[k].P = &P; wa[k].tid = k;
        pthread_create(&th[k], NULL, quality_worker, &wa[k]);
    }
    for (int k = 0; k < P.nthreads; k++) pthread_join(th[k], NULL);
    return 0;
}

/* One block score s^(l)_{t,i} for one query head: kind 0 the LSE of eq 21,
 * kind 1 / 2 the PISA-1 / PISA-2 scores of eq 33-34; exposed so tests can check
 * the score definitions themselves. q: d floats of one query head. */
double orc_score_kind(const float *q, int64_t b, int h, int l, int64_t i, const float *K,
                      const double *pyr, const int64_t *off, int B, int64_t N_alloc, int64_t N,
                      int H, int d, int C, int g, int kind)
{
    orc_problem P;
    int64_t zero = 0;
    if (kind < 0 || kind > 2) return NAN;
    if (setup(&P, q, &zero, &zero, 0, K, pyr, off, B, N_alloc, N, H, H, d, C, g, 3, 0, 1))
        return NAN;
    if (l < 1 || l > P.L || i < 0 || i >= P.M[l]) return NAN;
    P.score_kind = kind;
    return orc_lse_score(&P, b, h, q, l, i);
}

double orc_score(const float *q, int64_t b, int h, int l, int64_t i, const float *K,
                 const double *pyr, const int64_t *off, int B, int64_t N_alloc, int64_t N,
                 int H, int d, int C, int g)
{
    return orc_score_kind(q, b, h, l, i, K, pyr, off, B, N_alloc, N, H, d, C, g, 0);
}
