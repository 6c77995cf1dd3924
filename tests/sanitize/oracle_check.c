/*
 * The CPU oracle (oracle/tra_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every exported function on small inputs, ragged shapes and invalid arguments.  Built and
 * run by tests/test_sanitizers.py; any sanitizer report aborts with a non-zero status.
 * Prints "oracle sanitize ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_tile_major_order(int F, int H, int W, int th, int tw, int64_t *perm);
int orc_attention(const double *q, const double *k, const double *v, int N, int D, double scale,
                  const int32_t *rows, int nrows, const uint8_t *block_mask, int bq, int bk,
                  double *o, double *ent, double *lse, int nthreads);
double orc_token_budget(double H, double tau);
int orc_frame_norm(int F, double gamma, double *S);
double orc_base_radius(double H, double tau, double S_f);
int orc_lambda_table(int F, float tau, float gamma, double *lam);
int orc_log_table(int tmax, double *lnT);
int orc_member_row(const float *ent, int F, int H, int W, float tau, float gamma, int th, int tw, int i,
                   uint8_t *member);
int64_t orc_count_naive_disagreements(const float *ent, int F, int H, int W, float tau, float gamma, int th,
                                      int tw);
int orc_block_mask(const float *ent, int F, int H, int W, float tau, float gamma, int bq, int bk,
                   int vote_threshold, int th, int tw, const int32_t *qblocks, int nsel, uint8_t *mask,
                   int32_t *votes, int nthreads);
double orc_window_mu(float tau);
int orc_member_row_1d(const float *ent, int F, int H, int W, float tau, int th, int tw, int i, uint8_t *member);
int64_t orc_count_naive_disagreements_1d(const float *ent, int F, int H, int W, float tau, int th, int tw);
int orc_block_mask_1d(const float *ent, int F, int H, int W, float tau, int bq, int bk, int vote_threshold,
                      int th, int tw, const int32_t *qblocks, int nsel, uint8_t *mask, int32_t *votes,
                      int nthreads);

#define FAIL(msg)                                  \
    do {                                           \
        fprintf(stderr, "failed: %s\n", msg);      \
        return 1;                                  \
    } while (0)

static unsigned lcg_state = 7u;
static double urand(void) {
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (double)(lcg_state >> 8) / 16777216.0;
}

int main(void) {
    /* permutation: several shapes, clipped tiles, invalid arguments */
    const int shapes[][5] = {{1, 1, 1, 8, 8}, {2, 9, 7, 4, 3}, {3, 15, 17, 8, 8}, {1, 13, 11, 5, 4}};
    for (int s = 0; s < 4; ++s) {
        const int F = shapes[s][0], H = shapes[s][1], W = shapes[s][2];
        const int N = F * H * W;
        int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
        if (orc_tile_major_order(F, H, W, shapes[s][3], shapes[s][4], perm)) FAIL("tile_major_order");
        free(perm);
    }
    if (orc_tile_major_order(0, 4, 4, 8, 8, NULL) == 0) FAIL("tile_major_order accepted F = 0");

    /* attention: dense and block-masked, all rows and a subset, with a ragged block */
    {
        const int N = 100, D = 16, bq = 32, bk = 32, nqb = 4, nkb = 4;
        double *q = malloc(sizeof(double) * N * D), *k = malloc(sizeof(double) * N * D);
        double *v = malloc(sizeof(double) * N * D), *o = malloc(sizeof(double) * N * D);
        double *ent = malloc(sizeof(double) * N), *lse = malloc(sizeof(double) * N);
        int32_t rows[100];
        uint8_t mask[16];
        for (int i = 0; i < N * D; ++i) { q[i] = urand() - 0.5; k[i] = urand() - 0.5; v[i] = urand(); }
        for (int i = 0; i < N; ++i) rows[i] = i;
        for (int i = 0; i < nqb * nkb; ++i) mask[i] = (uint8_t)((i % 3) != 1);
        if (orc_attention(q, k, v, N, D, 0.25, rows, N, NULL, 0, 0, o, ent, lse, 3)) FAIL("dense attention");
        for (int i = 0; i < N; ++i)
            if (!(ent[i] >= -1e-12 && ent[i] <= log((double)N) + 1e-12)) FAIL("entropy range");
        if (orc_attention(q, k, v, N, D, 0.25, rows + 37, 11, mask, bq, bk, o, ent, lse, 2)) FAIL("masked attention");
        rows[0] = N;
        if (orc_attention(q, k, v, N, D, 0.25, rows, 1, NULL, 0, 0, o, ent, lse, 1) == 0) FAIL("row past N accepted");
        free(q); free(k); free(v); free(o); free(ent); free(lse);
    }

    /* budget, radius, tables */
    {
        double S[9], lam[81], lnT[200];
        if (orc_frame_norm(9, 0.5, S)) FAIL("frame_norm");
        if (!(orc_base_radius(3.0, 0.03, S[4]) > 0.0) || !(orc_token_budget(3.0, 0.03) > 0.0)) FAIL("radius");
        if (orc_lambda_table(9, 0.03f, 0.5f, lam)) FAIL("lambda_table");
        if (orc_log_table(199, lnT)) FAIL("log_table");
        if (orc_frame_norm(0, 0.5, S) == 0) FAIL("frame_norm accepted F = 0");
    }

    /* membership, naive-test agreement, block masks (ragged, several thresholds, special entropies) */
    {
        const int F = 3, H = 9, W = 11, N = F * H * W, bq = 64, bk = 64;
        const int nqb = (N + bq - 1) / bq, nkb = (N + bk - 1) / bk;
        float *ent = malloc(sizeof(float) * N);
        uint8_t *member = malloc((size_t)N);
        uint8_t *mask = malloc((size_t)nqb * nkb);
        int32_t *votes = malloc(sizeof(int32_t) * (size_t)nqb * nkb);
        int32_t qb[16];
        for (int i = 0; i < N; ++i) ent[i] = (float)(urand() * log((double)N));
        ent[0] = NAN; ent[1] = INFINITY; ent[2] = -INFINITY; ent[3] = -2.0f; ent[4] = 0.0f;
        for (int i = 0; i < nqb; ++i) qb[i] = i;
        if (orc_member_row(ent, F, H, W, 0.05f, 0.5f, 8, 8, N - 1, member)) FAIL("member_row");
        if (orc_member_row(ent, F, H, W, 0.05f, 0.5f, 8, 8, N, member) == 0) FAIL("member_row accepted i = N");
        if (orc_member_row(NULL, F, H, W, 0.05f, 0.5f, 8, 8, 0, member) == 0) FAIL("member_row accepted NULL");
        if (orc_count_naive_disagreements(ent + 5, 2, 6, 7, 0.1f, 0.3f, 4, 4) < 0) FAIL("naive disagreements");
        if (orc_count_naive_disagreements(NULL, 2, 6, 7, 0.1f, 0.3f, 4, 4) >= 0) FAIL("disagreements accepted NULL");
        for (int vote = 1; vote <= 3; ++vote)
            if (orc_block_mask(ent, F, H, W, 0.05f, 0.5f, bq, bk, vote, 8, 8, qb, nqb, mask, votes, 3))
                FAIL("block_mask");
        /* the 1D-window variant on the same entropies (NaN and infinities included) */
        if (!(orc_window_mu(0.5f) < 0.0)) FAIL("window_mu");
        if (orc_member_row_1d(ent, F, H, W, 0.05f, 4, 3, N - 1, member)) FAIL("member_row_1d");
        if (orc_member_row_1d(ent, F, H, W, 0.05f, 8, 8, N, member) == 0) FAIL("member_row_1d accepted i = N");
        if (orc_count_naive_disagreements_1d(ent + 5, 2, 6, 7, 0.1f, 4, 4) < 0) FAIL("naive disagreements 1d");
        if (orc_count_naive_disagreements_1d(NULL, 2, 6, 7, 0.1f, 4, 4) >= 0) FAIL("1d disagreements accepted NULL");
        for (int vote = 1; vote <= 3; ++vote)
            if (orc_block_mask_1d(ent, F, H, W, 0.05f, bq, bk, vote, 8, 8, qb, nqb, mask, votes, 3))
                FAIL("block_mask_1d");
        if (orc_block_mask_1d(ent, F, H, W, 0.0f, bq, bk, 1, 8, 8, qb, nqb, mask, votes, 1) == 0)
            FAIL("block_mask_1d accepted tau = 0");
        if (orc_member_row_1d(ent, 1, 1, 1, 0.5f, 8, 8, 0, member)) FAIL("member_row_1d, N = 1");
        qb[0] = nqb;
        if (orc_block_mask(ent, F, H, W, 0.05f, 0.5f, bq, bk, 1, 8, 8, qb, 1, mask, votes, 1) == 0)
            FAIL("block_mask accepted a q-block past the end");
        if (orc_block_mask_1d(ent, F, H, W, 0.05f, bq, bk, 1, 8, 8, qb, 1, mask, votes, 1) == 0)
            FAIL("block_mask_1d accepted a q-block past the end");
        free(ent); free(member); free(mask); free(votes);
    }
    printf("oracle sanitize ok\n");
    return 0;
}
