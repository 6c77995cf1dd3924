/*
 * tra_oracle.c -- plain, slow, fp64 CPU oracle for the Token Radius Attention
 * (TRA) hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  The product path
 * (the HIP library) never links, calls or includes anything here, and nothing
 * here includes or calls the HIP library: the two share no code.
 *
 * Every function writes out the plain definition of one step of the method as
 * the TRA pages state it ("Token Radius Attention for Efficient Video
 * Generation", gist.science summary of arXiv 2608.02504: section 2 "Method",
 * Insight I, Insight II and the TRA pipeline).  Where the pages leave a step
 * open, the reading adopted is stated in the comment of that function.
 *
 * Parity status: every function below is pinned by the CPU tests against
 * closed forms, invariants or brute force (tests/test_oracle_*.py).
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 *        -pthread -o liboracle.so tra_oracle.c -lm
 * (-ffp-contract=off keeps every fp64 operation a separately rounded step,
 * so that the threshold tables are reproducible bit for bit.)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* ------------------------------------------------------------------------- */
/* a tiny static-partition parallel-for over [0, n) with pthreads             */
/* ------------------------------------------------------------------------- */
typedef void (*orc_body)(void *ctx, int64_t lo, int64_t hi);
typedef struct { orc_body fn; void *ctx; int64_t lo, hi; } orc_slice;

static void *orc_slice_run(void *arg) {
    orc_slice *s = (orc_slice *)arg;
    if (s->lo < s->hi) s->fn(s->ctx, s->lo, s->hi);
    return NULL;
}

static void orc_parallel_for(int64_t n, int nthreads, orc_body fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t tid[256];
    orc_slice sl[256];
    for (int t = 0; t < nthreads; ++t) {
        sl[t].fn = fn; sl[t].ctx = ctx;
        sl[t].lo = n * t / nthreads; sl[t].hi = n * (t + 1) / nthreads;
        pthread_create(&tid[t], NULL, orc_slice_run, &sl[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Tile-major order (pipeline step 3, "tile-major layout": spatially          */
/* neighbouring tokens are made contiguous in the sequence).                  */
/*                                                                           */
/* Reading: tokens are natural-indexed (f*H + h)*W + w.  Tile-major order     */
/* visits frame f, then rows of tiles, then tiles left to right, then the     */
/* rows inside a tile, then the columns inside a tile.  Tiles are th x tw;    */
/* tiles on the bottom and right edges are clipped, nothing is padded.        */
/* This function ENUMERATES that order with nested loops (no closed form):    */
/* perm[p] = natural index of the token at tile-major position p.            */
/* ------------------------------------------------------------------------- */
int orc_tile_major_order(int F, int H, int W, int th, int tw, int64_t *perm) {
    if (F < 1 || H < 1 || W < 1 || th < 1 || tw < 1 || !perm) return 1;
    int64_t p = 0;
    for (int f = 0; f < F; ++f)
        for (int y0 = 0; y0 < H; y0 += th)
            for (int x0 = 0; x0 < W; x0 += tw)
                for (int y = y0; y < y0 + th && y < H; ++y)
                    for (int x = x0; x < x0 + tw && x < W; ++x)
                        perm[p++] = ((int64_t)f * H + y) * W + x;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Attention and per-query entropy (section 1: dense 3D self-attention over   */
/* the N video tokens; pipeline step 1: the per-query attention entropy taken */
/* during the dense warm-up; Insight I: entropy of the attention row).        */
/*                                                                           */
/* s_ij = scale * <q_i, k_j>; p_i = softmax over the allowed keys of row i;   */
/* o_i = sum_j p_ij v_j; H_i = -sum_j p_ij ln p_ij (nats, 0 ln 0 = 0);        */
/* lse_i = ln sum_j exp(s_ij).  Two passes, fp64, straight from the           */
/* definition.  Non-causal.                                                   */
/*                                                                           */
/* Allowed keys: all N keys when block_mask is NULL (dense).  Otherwise the   */
/* block-sparse reading: row i (a position in the given order) lives in       */
/* q-block i / bq, key j in k-block j / bk, and j is allowed iff              */
/* block_mask[(i / bq) * nkb + j / bk] != 0 -- every token of a retained      */
/* block and nothing else (pipeline step 3: the token mask becomes a regular  */
/* block-sparse mask that an existing block-sparse backend executes).         */
/* ------------------------------------------------------------------------- */
typedef struct {
    const double *q, *k, *v;
    int N, D;
    double scale;
    const int32_t *rows;
    const uint8_t *block_mask;
    int bq, bk, nkb;
    double *o, *ent, *lse;
} orc_attn_ctx;

static void orc_attn_body(void *vctx, int64_t lo, int64_t hi) {
    orc_attn_ctx *c = (orc_attn_ctx *)vctx;
    const int N = c->N, D = c->D;
    double *s = (double *)malloc(sizeof(double) * (size_t)N);
    uint8_t *ok = (uint8_t *)malloc((size_t)N);
    for (int64_t r = lo; r < hi; ++r) {
        const int i = c->rows[r];
        const double *qi = c->q + (int64_t)i * D;
        for (int j = 0; j < N; ++j) {
            ok[j] = 1;
            if (c->block_mask)
                ok[j] = c->block_mask[(int64_t)(i / c->bq) * c->nkb + j / c->bk] != 0;
        }
        /* pass 1: scores and their maximum */
        double mx = -INFINITY;
        for (int j = 0; j < N; ++j) {
            if (!ok[j]) continue;
            const double *kj = c->k + (int64_t)j * D;
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += qi[d] * kj[d];
            s[j] = c->scale * acc;
            if (s[j] > mx) mx = s[j];
        }
        /* pass 2: normaliser */
        double z = 0.0;
        for (int j = 0; j < N; ++j)
            if (ok[j]) z += exp(s[j] - mx);
        /* probabilities, output, entropy */
        double *oi = c->o + r * D;
        for (int d = 0; d < D; ++d) oi[d] = 0.0;
        double h = 0.0;
        for (int j = 0; j < N; ++j) {
            if (!ok[j]) continue;
            const double p = exp(s[j] - mx) / z;
            const double *vj = c->v + (int64_t)j * D;
            for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
            if (p > 0.0) h -= p * log(p);
        }
        if (c->ent) c->ent[r] = h;
        if (c->lse) c->lse[r] = mx + log(z);
    }
    free(s);
    free(ok);
}

int orc_attention(const double *q, const double *k, const double *v, int N, int D, double scale,
                  const int32_t *rows, int nrows, const uint8_t *block_mask, int bq, int bk,
                  double *o, double *ent, double *lse, int nthreads) {
    if (!q || !k || !v || !rows || !o || N < 1 || D < 1 || nrows < 0) return 1;
    if (block_mask && (bq < 1 || bk < 1)) return 1;
    for (int r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return 1;
    orc_attn_ctx c = {q, k, v, N, D, scale, rows, block_mask, bq, bk,
                      block_mask ? (N + bk - 1) / bk : 0, o, ent, lse};
    orc_parallel_for(nrows, nthreads, orc_attn_body, &c);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Entropy -> budget -> radius (Insight I: budget B = tau * exp(H_i) / N as a */
/* fraction of the N keys; Insight II: the budget becomes a query-specific    */
/* base radius, scaled per frame by phi(delta) = exp(-gamma * delta) with     */
/* delta the temporal distance; pipeline step 2: a 2D disk per frame).        */
/*                                                                           */
/* Readings (the pages give the two formulas and no more):                   */
/*  - token budget K_i = B * N = tau * exp(H_i), no clamp;                   */
/*  - phi scales the RADIUS: rho_i(f') = r_i * exp(-gamma |f_i - f'|);        */
/*  - r_i is fixed by area matching over the frames present:                  */
/*      sum_f' pi * rho_i(f')^2 = K_i  =>  r_i^2 = K_i / (pi * S_{f_i}),      */
/*      S_f = sum_{f'=0}^{F-1} exp(-2 gamma |f - f'|)  (summed in increasing f');*/
/*  - key j belongs to query i's support iff                                  */
/*      (h_i - h_j)^2 + (w_i - w_j)^2 <= rho_i(f_j)^2                          */
/*    (Euclidean distance in latent tokens, inclusive, no wrap, all frames).  */
/*  - canonical evaluation, so that a fixed rule decides every case bit for   */
/*    bit: with d2 = squared distance, j is a member iff d2 == 0 or           */
/*      ln(d2) <= (double)H_i + lambda[f_i][f_j],                             */
/*      lambda[f][f'] = (ln tau - (2 gamma) |f - f'|) - ln(pi * S_f),          */
/*    ln(d2) taken from a table of ln t for t = 1..(H-1)^2+(W-1)^2, all in    */
/*    fp64 with the C library's log and exp, in exactly this operation order. */
/*    This is the log of the disk inequality above.                           */
/* ------------------------------------------------------------------------- */

/* K_i = tau * exp(H_i): the budget in tokens */
double orc_token_budget(double H, double tau) { return tau * exp(H); }

/* S_f for every frame f, summed over f' in increasing order */
int orc_frame_norm(int F, double gamma, double *S) {
    if (F < 1 || !S) return 1;
    for (int f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int fp = 0; fp < F; ++fp) {
            const int delta = f > fp ? f - fp : fp - f;
            acc += exp(-(2.0 * gamma) * (double)delta);
        }
        S[f] = acc;
    }
    return 0;
}

/* base radius r_i = sqrt(K_i / (pi * S_f)) (area matching) */
double orc_base_radius(double H, double tau, double S_f) {
    return sqrt(orc_token_budget(H, tau) / (M_PI * S_f));
}

/* lambda[f * F + f'] = (ln tau - (2 gamma) |f - f'|) - ln(pi * S_f) */
int orc_lambda_table(int F, float tau, float gamma, double *lam) {
    if (F < 1 || !lam || !(tau > 0.0f) || !(gamma >= 0.0f)) return 1;
    const double t = (double)tau, g = (double)gamma;
    double *S = (double *)malloc(sizeof(double) * (size_t)F);
    orc_frame_norm(F, g, S);
    for (int f = 0; f < F; ++f)
        for (int fp = 0; fp < F; ++fp) {
            const int delta = f > fp ? f - fp : fp - f;
            lam[(int64_t)f * F + fp] = (log(t) - (2.0 * g) * (double)delta) - log(M_PI * S[f]);
        }
    free(S);
    return 0;
}

/* lnT[t] = ln t for t = 1..tmax; lnT[0] is unused and set to -inf */
int orc_log_table(int tmax, double *lnT) {
    if (tmax < 0 || !lnT) return 1;
    lnT[0] = -INFINITY;
    for (int t = 1; t <= tmax; ++t) lnT[t] = log((double)t);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Geometry shared by the mask functions                                      */
/* ------------------------------------------------------------------------- */
typedef struct {
    int F, H, W, N, th, tw;
    int32_t *fr, *hy, *wx; /* coordinates of the token at each tile-major position */
    double *lam;           /* [F][F] */
    double *lnT;           /* [tmax + 1] */
    int tmax;
} orc_geom;

static int orc_geom_init(orc_geom *g, int F, int H, int W, int th, int tw, float tau, float gamma) {
    memset(g, 0, sizeof(*g));
    if (F < 1 || H < 1 || W < 1 || th < 1 || tw < 1) return 1;
    g->F = F; g->H = H; g->W = W; g->th = th; g->tw = tw;
    g->N = F * H * W;
    g->tmax = (H - 1) * (H - 1) + (W - 1) * (W - 1);
    int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)g->N);
    g->fr = (int32_t *)malloc(sizeof(int32_t) * (size_t)g->N);
    g->hy = (int32_t *)malloc(sizeof(int32_t) * (size_t)g->N);
    g->wx = (int32_t *)malloc(sizeof(int32_t) * (size_t)g->N);
    g->lam = (double *)malloc(sizeof(double) * (size_t)F * F);
    g->lnT = (double *)malloc(sizeof(double) * (size_t)(g->tmax + 1));
    if (!perm || !g->fr || !g->hy || !g->wx || !g->lam || !g->lnT) {
        free(perm);
        return 1;
    }
    orc_tile_major_order(F, H, W, th, tw, perm);
    for (int p = 0; p < g->N; ++p) {
        const int64_t n = perm[p];
        g->fr[p] = (int32_t)(n / ((int64_t)H * W));
        g->hy[p] = (int32_t)((n / W) % H);
        g->wx[p] = (int32_t)(n % W);
    }
    free(perm);
    if (orc_lambda_table(F, tau, gamma, g->lam)) return 1;
    orc_log_table(g->tmax, g->lnT);
    return 0;
}

static void orc_geom_free(orc_geom *g) {
    free(g->fr); free(g->hy); free(g->wx); free(g->lam); free(g->lnT);
    memset(g, 0, sizeof(*g));
}

/* canonical membership: is the key at tile-major position j in the support
 * of the query at tile-major position i whose entropy is Hi? */
static int orc_is_member(const orc_geom *g, float Hi, int i, int j) {
    const int dh = g->hy[i] - g->hy[j], dw = g->wx[i] - g->wx[j];
    const int d2 = dh * dh + dw * dw;
    if (d2 == 0) return 1;
    const double s = (double)Hi + g->lam[(int64_t)g->fr[i] * g->F + g->fr[j]];
    return g->lnT[d2] <= s;
}

/* the same disk written directly as a radius test in fp64 (no tables):
 * d2 <= (r_i * exp(-gamma * delta))^2 with r_i the area-matched base radius */
static int orc_is_member_naive(const orc_geom *g, const double *S, float Hi, float tau, float gamma,
                               int i, int j) {
    const int dh = g->hy[i] - g->hy[j], dw = g->wx[i] - g->wx[j];
    const int d2 = dh * dh + dw * dw;
    const int fi = g->fr[i], fj = g->fr[j];
    const int delta = fi > fj ? fi - fj : fj - fi;
    const double r = orc_base_radius((double)Hi, (double)tau, S[fi]);
    const double rho = r * exp(-(double)gamma * (double)delta);
    return (double)d2 <= rho * rho;
}

/* ------------------------------------------------------------------------- */
/* 1D-distance support (section 4, ablation study: the radius mask replaced   */
/* by a 1D distance).                                                         */
/*                                                                           */
/* Reading (the pages name the variant and nothing more): the same token      */
/* budget K_i = tau * exp(H_i) is spent on a window of the flattened token    */
/* sequence in its natural raster order n = (f*H + h)*W + w, centred on the   */
/* query: key j belongs to the support iff                                   */
/*     2 |n_i - n_j| <= K_i,                                                 */
/* so the window holds about K_i keys (the 1D counterpart of area matching).  */
/* No per-frame factor: the 1D sequence has no frame axis.  Canonical        */
/* evaluation, as for the disk: with d = |n_i - n_j|, j is a member iff       */
/* d == 0 or ln(d) <= (double)H_i + mu, mu = ln tau - ln 2, ln(d) from a      */
/* table of ln t for t = 1..N-1 -- the log of the window inequality, fp64,    */
/* with the C library's log.                                                 */
/* ------------------------------------------------------------------------- */

/* mu = ln tau - ln 2 */
double orc_window_mu(float tau) { return log((double)tau) - log(2.0); }

static int64_t orc_natural_index(const orc_geom *g, int p) {
    return ((int64_t)g->fr[p] * g->H + g->hy[p]) * g->W + g->wx[p];
}

/* canonical window membership of the key at tile-major position j for the
 * query at tile-major position i; lnT1 has N entries (ln t, t < N) */
static int orc_is_member_1d(const orc_geom *g, const double *lnT1, double mu, float Hi, int i, int j) {
    const int64_t a = orc_natural_index(g, i), b = orc_natural_index(g, j);
    const int64_t d = a > b ? a - b : b - a;
    if (d == 0) return 1;
    return lnT1[d] <= (double)Hi + mu;
}

/* the same window written directly, fp64, no tables: 2 d <= tau * exp(H_i) */
static int orc_is_member_1d_naive(const orc_geom *g, float Hi, float tau, int i, int j) {
    const int64_t a = orc_natural_index(g, i), b = orc_natural_index(g, j);
    const int64_t d = a > b ? a - b : b - a;
    return 2.0 * (double)d <= orc_token_budget((double)Hi, (double)tau);
}

static double *orc_log_table_upto(int n) {
    double *t = (double *)malloc(sizeof(double) * (size_t)(n > 1 ? n : 1));
    if (t) orc_log_table(n - 1 > 0 ? n - 1 : 0, t);
    return t;
}

/* Window support of one query (all N keys, tile-major positions). */
int orc_member_row_1d(const float *ent, int F, int H, int W, float tau, int th, int tw, int i, uint8_t *member) {
    orc_geom g = {0};
    if (!ent || !member || orc_geom_init(&g, F, H, W, th, tw, tau, 0.0f)) { orc_geom_free(&g); return 1; }
    if (i < 0 || i >= g.N) { orc_geom_free(&g); return 1; }
    double *lnT1 = orc_log_table_upto(g.N);
    if (!lnT1) { orc_geom_free(&g); return 1; }
    const double mu = orc_window_mu(tau);
    for (int j = 0; j < g.N; ++j) member[j] = (uint8_t)orc_is_member_1d(&g, lnT1, mu, ent[i], i, j);
    free(lnT1);
    orc_geom_free(&g);
    return 0;
}

/* Pairs on which the canonical window test and the direct fp64 test disagree
 * (all N*N pairs; tiny grids only). */
int64_t orc_count_naive_disagreements_1d(const float *ent, int F, int H, int W, float tau, int th, int tw) {
    orc_geom g = {0};
    if (!ent || orc_geom_init(&g, F, H, W, th, tw, tau, 0.0f)) { orc_geom_free(&g); return -1; }
    double *lnT1 = orc_log_table_upto(g.N);
    if (!lnT1) { orc_geom_free(&g); return -1; }
    const double mu = orc_window_mu(tau);
    int64_t bad = 0;
    for (int i = 0; i < g.N; ++i)
        for (int j = 0; j < g.N; ++j)
            bad += orc_is_member_1d(&g, lnT1, mu, ent[i], i, j) != orc_is_member_1d_naive(&g, ent[i], tau, i, j);
    free(lnT1);
    orc_geom_free(&g);
    return bad;
}

/* Support of one query (all N keys, tile-major positions): member[j] in {0,1}.
 * ent: fp32 entropies in tile-major order. */
int orc_member_row(const float *ent, int F, int H, int W, float tau, float gamma, int th, int tw,
                   int i, uint8_t *member) {
    orc_geom g = {0};  /* freed on every exit, also before orc_geom_init runs */
    if (!ent || !member || orc_geom_init(&g, F, H, W, th, tw, tau, gamma)) { orc_geom_free(&g); return 1; }
    if (i < 0 || i >= g.N) { orc_geom_free(&g); return 1; }
    for (int j = 0; j < g.N; ++j) member[j] = (uint8_t)orc_is_member(&g, ent[i], i, j);
    orc_geom_free(&g);
    return 0;
}

/* Number of (query, key) pairs on which the canonical table test and the
 * direct fp64 radius test disagree, over all N*N pairs (tiny grids only). */
int64_t orc_count_naive_disagreements(const float *ent, int F, int H, int W, float tau, float gamma,
                                      int th, int tw) {
    orc_geom g = {0};  /* freed on every exit, also before orc_geom_init runs */
    if (!ent || orc_geom_init(&g, F, H, W, th, tw, tau, gamma)) { orc_geom_free(&g); return -1; }
    double *S = (double *)malloc(sizeof(double) * (size_t)F);
    orc_frame_norm(F, (double)gamma, S);
    int64_t bad = 0;
    for (int i = 0; i < g.N; ++i)
        for (int j = 0; j < g.N; ++j)
            bad += orc_is_member(&g, ent[i], i, j) != orc_is_member_naive(&g, S, ent[i], tau, gamma, i, j);
    free(S);
    orc_geom_free(&g);
    return bad;
}

/* ------------------------------------------------------------------------- */
/* Token-level mask -> block-sparse mask (pipeline step 3: distance           */
/* computation, radius comparison, block pruning and token voting turn the    */
/* irregular token-level radius mask into a regular block-sparse mask).       */
/*                                                                           */
/* Readings: blocks are contiguous ranges of the tile-major sequence, q-block */
/* b = [b*bq, min(N, (b+1)*bq)), k-blocks likewise with bk (ragged last       */
/* blocks).  Token voting: votes(Qb, Kb) = number of queries i in Qb whose    */
/* support meets Kb.  Kb is retained iff votes >= vote_threshold, or Kb       */
/* overlaps Qb's own index range (the diagonal is always kept).  Block        */
/* pruning is only a speed-up and cannot change this result, so the oracle    */
/* does no pruning: it tests every (query, key) pair.                          */
/*                                                                           */
/* Outputs for each selected q-block s (qblocks[s]): mask[s * nkb + kb] in    */
/* {0,1} and votes[s * nkb + kb].                                              */
/* ------------------------------------------------------------------------- */
typedef struct {
    const orc_geom *g;
    const float *ent;
    int bq, bk, nkb, vote;
    const int32_t *qblocks;
    uint8_t *mask;
    int32_t *votes;
    const double *lnT1; /* non-NULL: the 1D window support (orc_is_member_1d) instead of the disk */
    double mu;
} orc_mask_ctx;

static int orc_mask_member(const orc_mask_ctx *c, int i, int j) {
    if (c->lnT1) return orc_is_member_1d(c->g, c->lnT1, c->mu, c->ent[i], i, j);
    return orc_is_member(c->g, c->ent[i], i, j);
}

static void orc_mask_body(void *vctx, int64_t lo, int64_t hi) {
    orc_mask_ctx *c = (orc_mask_ctx *)vctx;
    const orc_geom *g = c->g;
    uint8_t *touched = (uint8_t *)malloc((size_t)c->nkb);
    for (int64_t s = lo; s < hi; ++s) {
        const int qb = c->qblocks[s];
        const int q0 = qb * c->bq;
        const int q1 = q0 + c->bq < g->N ? q0 + c->bq : g->N;
        int32_t *vt = c->votes + s * c->nkb;
        uint8_t *mk = c->mask + s * c->nkb;
        for (int kb = 0; kb < c->nkb; ++kb) vt[kb] = 0;
        for (int i = q0; i < q1; ++i) {
            memset(touched, 0, (size_t)c->nkb);
            for (int j = 0; j < g->N; ++j)
                if (orc_mask_member(c, i, j)) touched[j / c->bk] = 1;
            for (int kb = 0; kb < c->nkb; ++kb) vt[kb] += touched[kb];
        }
        for (int kb = 0; kb < c->nkb; ++kb) {
            const int k0 = kb * c->bk;
            const int k1 = k0 + c->bk < g->N ? k0 + c->bk : g->N;
            const int diagonal = k0 < q1 && q0 < k1;
            mk[kb] = (uint8_t)(vt[kb] >= c->vote || diagonal);
        }
    }
    free(touched);
}

int orc_block_mask(const float *ent, int F, int H, int W, float tau, float gamma, int bq, int bk,
                   int vote_threshold, int th, int tw, const int32_t *qblocks, int nsel,
                   uint8_t *mask, int32_t *votes, int nthreads) {
    orc_geom g = {0};  /* freed on every exit, also before orc_geom_init runs */
    if (!ent || !qblocks || !mask || !votes || bq < 1 || bk < 1 || vote_threshold < 1 || nsel < 0)
        return 1;
    if (orc_geom_init(&g, F, H, W, th, tw, tau, gamma)) { orc_geom_free(&g); return 1; }
    const int nqb = (g.N + bq - 1) / bq;
    for (int s = 0; s < nsel; ++s)
        if (qblocks[s] < 0 || qblocks[s] >= nqb) { orc_geom_free(&g); return 1; }
    orc_mask_ctx c = {&g, ent, bq, bk, (g.N + bk - 1) / bk, vote_threshold, qblocks, mask, votes, NULL, 0.0};
    orc_parallel_for(nsel, nthreads, orc_mask_body, &c);
    orc_geom_free(&g);
    return 0;
}

/* The same block voting over the 1D window support (ablation variant): mask
 * and votes of the selected q-blocks. */
int orc_block_mask_1d(const float *ent, int F, int H, int W, float tau, int bq, int bk, int vote_threshold,
                      int th, int tw, const int32_t *qblocks, int nsel, uint8_t *mask, int32_t *votes,
                      int nthreads) {
    orc_geom g = {0};
    if (!ent || !qblocks || !mask || !votes || bq < 1 || bk < 1 || vote_threshold < 1 || nsel < 0)
        return 1;
    if (!(tau > 0.0f)) return 1;
    if (orc_geom_init(&g, F, H, W, th, tw, tau, 0.0f)) { orc_geom_free(&g); return 1; }
    const int nqb = (g.N + bq - 1) / bq;
    for (int s = 0; s < nsel; ++s)
        if (qblocks[s] < 0 || qblocks[s] >= nqb) { orc_geom_free(&g); return 1; }
    double *lnT1 = orc_log_table_upto(g.N);
    if (!lnT1) { orc_geom_free(&g); return 1; }
    orc_mask_ctx c = {&g, ent, bq, bk, (g.N + bk - 1) / bk, vote_threshold, qblocks, mask, votes, lnT1,
                      orc_window_mu(tau)};
    orc_parallel_for(nsel, nthreads, orc_mask_body, &c);
    free(lnT1);
    orc_geom_free(&g);
    return 0;
}
