/*
 * A plain C99 caller of libtra.so (no Python, no torch): device buffers from the HIP
 * runtime, the TRA hot path through the C ABI of include/tra.h, results checked on the
 * host.  Built by the package's build step; run by tests/test_gpu_c_abi.py.
 *
 *   1. permute then unpermute restores q bit for bit;
 *   2. dense attention + entropy on the permuted tensors (entropies in [0, ln N]);
 *   3. a mask that keeps every block (tau large, gamma 0) lists every k-block in order;
 *   4. block-sparse attention over that mask equals the dense output bit for bit;
 *   5. an unsupported head size is refused with TRA_ERR_UNSUPPORTED before any work.
 * Prints "c abi ok" and exits 0, or names the failed check and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tra.h"

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            return 1;                                                           \
        }                                                                       \
    } while (0)

#define CHECK_TRA(x)                                                            \
    do {                                                                        \
        tra_status s_ = (x);                                                    \
        if (s_ != TRA_OK) {                                                     \
            fprintf(stderr, "%s at %s:%d\n", tra_status_string(s_), __FILE__, __LINE__); \
            return 1;                                                           \
        }                                                                       \
    } while (0)

static uint32_t lcg(uint32_t *s) {
    *s = *s * 1664525u + 1013904223u;
    return *s;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int main(void) {
    enum { OUTER = 2, F = 3, H = 8, W = 12, D = 128, BQ = 128, BK = 64 };
    const int N = F * H * W;
    const int nqb = (N + BQ - 1) / BQ, nkb = (N + BK - 1) / BK;
    const size_t elems = (size_t)OUTER * N * D, bytes = elems * 2;
    const float scale = 1.0f / sqrtf((float)D);

    uint16_t *h = (uint16_t *)malloc(3 * bytes), *h2 = (uint16_t *)malloc(2 * bytes);
    float *hent = (float *)malloc((size_t)OUTER * N * sizeof(float));
    int32_t *hcnt = (int32_t *)malloc((size_t)OUTER * nqb * sizeof(int32_t));
    int32_t *hidx = (int32_t *)malloc((size_t)OUTER * nqb * nkb * sizeof(int32_t));
    if (!h || !h2 || !hent || !hcnt || !hidx) return 1;
    uint32_t seed = 12345u;
    for (size_t i = 0; i < 3 * elems; ++i) {
        const float r = ((float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f) * 4.0f;
        h[i] = to_bf16(r);
    }

    void *q, *k, *v, *qp, *kp, *vp, *o, *os, *back;
    float *ent, *lse;
    int32_t *cnt, *idx;
    CHECK_HIP(hipMalloc(&q, bytes)); CHECK_HIP(hipMalloc(&k, bytes)); CHECK_HIP(hipMalloc(&v, bytes));
    CHECK_HIP(hipMalloc(&qp, bytes)); CHECK_HIP(hipMalloc(&kp, bytes)); CHECK_HIP(hipMalloc(&vp, bytes));
    CHECK_HIP(hipMalloc(&o, bytes)); CHECK_HIP(hipMalloc(&os, bytes)); CHECK_HIP(hipMalloc(&back, bytes));
    CHECK_HIP(hipMalloc((void **)&ent, (size_t)OUTER * N * sizeof(float)));
    CHECK_HIP(hipMalloc((void **)&lse, (size_t)OUTER * N * sizeof(float)));
    CHECK_HIP(hipMalloc((void **)&cnt, (size_t)OUTER * nqb * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void **)&idx, (size_t)OUTER * nqb * nkb * sizeof(int32_t)));
    CHECK_HIP(hipMemcpy(q, h, bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(k, h + elems, bytes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, h + 2 * elems, bytes, hipMemcpyHostToDevice));

    /* 1. permutation round trip */
    CHECK_TRA(tra_tile_major_permute(q, qp, OUTER, F, H, W, D, TRA_BF16, 8, 8, 0));
    CHECK_TRA(tra_tile_major_permute(k, kp, OUTER, F, H, W, D, TRA_BF16, 8, 8, 0));
    CHECK_TRA(tra_tile_major_permute(v, vp, OUTER, F, H, W, D, TRA_BF16, 8, 8, 0));
    CHECK_TRA(tra_tile_major_unpermute(qp, back, OUTER, F, H, W, D, TRA_BF16, 8, 8, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(h2, back, bytes, hipMemcpyDeviceToHost));
    if (memcmp(h2, h, bytes) != 0) {
        fprintf(stderr, "check 1: permute round trip differs\n");
        return 1;
    }

    /* 2. dense attention + entropy */
    CHECK_TRA(tra_dense_attn_entropy(qp, kp, vp, o, ent, lse, OUTER, N, D, TRA_BF16, scale, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hent, ent, (size_t)OUTER * N * sizeof(float), hipMemcpyDeviceToHost));
    for (int i = 0; i < OUTER * N; ++i)
        if (!(hent[i] >= -1e-3f && hent[i] <= logf((float)N) + 1e-3f)) {
            fprintf(stderr, "check 2: entropy %d = %g outside [0, ln N]\n", i, hent[i]);
            return 1;
        }

    /* 3. a mask that keeps every block */
    CHECK_TRA(tra_build_block_mask(ent, OUTER, F, H, W, 1.0e6f, 0.0f, BQ, BK, 1, 8, 8, cnt, idx,
                                   (int64_t)OUTER * nqb * nkb, NULL, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hcnt, cnt, (size_t)OUTER * nqb * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hidx, idx, (size_t)OUTER * nqb * nkb * sizeof(int32_t), hipMemcpyDeviceToHost));
    for (int r = 0; r < OUTER * nqb; ++r) {
        if (hcnt[r] != nkb) {
            fprintf(stderr, "check 3: row %d keeps %d of %d k-blocks\n", r, hcnt[r], nkb);
            return 1;
        }
        for (int j = 0; j < nkb; ++j)
            if (hidx[(size_t)r * nkb + j] != j) {
                fprintf(stderr, "check 3: row %d entry %d = %d\n", r, j, hidx[(size_t)r * nkb + j]);
                return 1;
            }
    }

    /* 4. sparse over every block = dense, bit for bit */
    CHECK_TRA(tra_block_sparse_attn(qp, kp, vp, os, NULL, cnt, idx, OUTER, N, D, TRA_BF16, scale, BQ, BK, 0));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(h2, o, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h2 + elems, os, bytes, hipMemcpyDeviceToHost));
    if (memcmp(h2, h2 + elems, bytes) != 0) {
        fprintf(stderr, "check 4: sparse over every block differs from dense\n");
        return 1;
    }

    /* 5. unsupported head size: refused before any HIP call */
    if (tra_block_sparse_attn(qp, kp, vp, os, NULL, cnt, idx, OUTER, N, 96, TRA_BF16, scale, BQ, BK, 0) !=
        TRA_ERR_UNSUPPORTED) {
        fprintf(stderr, "check 5: D = 96 was not refused\n");
        return 1;
    }

    hipFree(q); hipFree(k); hipFree(v); hipFree(qp); hipFree(kp); hipFree(vp);
    hipFree(o); hipFree(os); hipFree(back); hipFree(ent); hipFree(lse); hipFree(cnt); hipFree(idx);
    free(h); free(h2); free(hent); free(hcnt); free(hidx);
    printf("c abi ok\n");
    return 0;
}
