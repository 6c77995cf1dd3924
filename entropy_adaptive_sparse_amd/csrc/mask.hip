// mask.hip -- entropy -> budget -> radius -> block-sparse mask, one fused kernel
// ("Token Radius Attention for Efficient Video Generation", section 2: Insight I
// budget tau * exp(H_i) / N; Insight II radius with per-frame factor
// exp(-gamma * delta); TRA pipeline steps 2-3: a 2D disk per frame, then distance
// computation, radius comparison, block pruning and token voting fused into one
// kernel that emits a regular block-sparse mask).
//
// One workgroup per (head, q-block):
//  1. thresholds: for each query i of the q-block and each frame f', the largest
//     squared distance the disk admits, T_i(f') = max{t : t = 0 or ln t <= s},
//     s = (double)H_i + lambda[f_i][f'] (one fp64 add; ln t from a host-built fp64
//     table, so no transcendental decides anything on the device).  Kept in LDS.
//  2. block pruning: a k-block is a union of axis-aligned rectangles (host table);
//     the squared distance from the q-block's bounding box to a rectangle bounds
//     every query's distance from below, so a rectangle that lies beyond the
//     q-block's largest threshold for its frame cannot receive a vote.
//  3. token voting on the surviving k-blocks: one wavefront per k-block, one lane
//     per query (two for 128-query blocks); a lane votes if its disk meets any
//     rectangle (exact: the nearest lattice point of a rectangle is the clamped
//     query position); the block's vote count is the popcount of the ballot.
//  4. compaction: retained k-blocks are written as an ascending index list with a
//     workgroup prefix sum, plus the count and the optional byte mask.
#include "tra_internal.h"

#include <climits>

namespace tra {

namespace {

constexpr int kThreads = 256;

__device__ inline int threshold_from(double s, const double *__restrict__ lnT, int tmax) {
    if (!(s >= 0.0) || tmax == 0) return 0;  // s < ln 1 (or NaN): only the query's own position
    if (s >= lnT[tmax]) return tmax;         // the whole frame
    int t = (int)__expf((float)s);           // a guess; the table decides below
    t = max(1, min(t, tmax));
    while (t < tmax && lnT[t + 1] <= s) ++t;
    while (t > 1 && lnT[t] > s) --t;
    return t;
}

__device__ inline int rect_dist2(int4 r, int h, int w) {
    const int y0 = r.y & 0xffff, y1 = r.y >> 16;
    const int x0 = r.z & 0xffff, x1 = r.z >> 16;
    const int dh = max(0, max(y0 - h, h - y1));
    const int dw = max(0, max(x0 - w, w - x1));
    return dh * dh + dw * dw;
}

__global__ __launch_bounds__(kThreads) void build_mask_kernel(MaskArgs a) {
    extern __shared__ int smem[];
    const int BQ = a.block_q, F = a.g.F, nkb = a.nkb, N = a.g.N;
    int *sT = smem;              // [BQ][F]
    int *sTmax = sT + BQ * F;    // [F]
    int *sqf = sTmax + F;        // [BQ]
    int *sqh = sqf + BQ;         // [BQ]
    int *sqw = sqh + BQ;         // [BQ]
    float *sH = (float *)(sqw + BQ);  // [BQ]
    int *scand = (int *)(sH + BQ);    // [nkb]
    int *sscan = scand + nkb;    // [kThreads]
    int *sbox = sscan + kThreads;     // hmin hmax wmin wmax ncand
    unsigned char *sflag = (unsigned char *)(sbox + 8);  // [nkb]

    const int tid = threadIdx.x;
    const int o = blockIdx.x / a.nqb;
    const int qb = blockIdx.x - o * a.nqb;
    const int q0 = qb * BQ;
    const int nq = min(BQ, N - q0);
    const float *ent = a.ent + (int64_t)o * N;

    if (tid == 0) {
        sbox[0] = INT_MAX; sbox[1] = INT_MIN; sbox[2] = INT_MAX; sbox[3] = INT_MIN; sbox[4] = 0;
    }
    for (int f = tid; f < F; f += kThreads) sTmax[f] = 0;
    __syncthreads();

    // query coordinates, entropies and the q-block's bounding box
    for (int i = tid; i < nq; i += kThreads) {
        int f, y, x;
        tile_major_coords(q0 + i, a.g, f, y, x);
        sqf[i] = f; sqh[i] = y; sqw[i] = x;
        sH[i] = ent[q0 + i];
        atomicMin(&sbox[0], y); atomicMax(&sbox[1], y);
        atomicMin(&sbox[2], x); atomicMax(&sbox[3], x);
    }
    __syncthreads();

    // 1. per-(query, frame) integer thresholds
    for (int idx = tid; idx < nq * F; idx += kThreads) {
        const int i = idx / F;
        const int fp = idx - i * F;
        const double s = (double)sH[i] + a.t.lam[sqf[i] * F + fp];
        const int T = threshold_from(s, a.t.lnT, a.t.tmax);
        sT[idx] = T;
        atomicMax(&sTmax[fp], T);
    }
    __syncthreads();

    // 2. diagonal guard and block pruning; surviving k-blocks become candidates
    const int hmin = sbox[0], hmax = sbox[1], wmin = sbox[2], wmax = sbox[3];
    for (int kb = tid; kb < nkb; kb += kThreads) {
        const int k0 = kb * a.block_k;
        const int k1 = min(N, k0 + a.block_k);
        int flag = 0;
        if (k0 < q0 + nq && q0 < k1) {
            flag = 1;
        } else {
            const int r1 = a.t.rect_off[kb + 1];
            for (int r = a.t.rect_off[kb]; r < r1; ++r) {
                const int4 rc = a.t.rects[r];
                const int y0 = rc.y & 0xffff, y1 = rc.y >> 16;
                const int x0 = rc.z & 0xffff, x1 = rc.z >> 16;
                const int dh = max(0, max(y0 - hmax, hmin - y1));
                const int dw = max(0, max(x0 - wmax, wmin - x1));
                if (dh * dh + dw * dw <= sTmax[rc.x]) { flag = 2; break; }
            }
        }
        sflag[kb] = (unsigned char)flag;
        if (flag == 2) scand[atomicAdd(&sbox[4], 1)] = kb;
    }
    __syncthreads();

    // 3. token voting, one wavefront per candidate k-block
    const int lane = tid & 63, wave = tid >> 6;
    const int ncand = sbox[4];
    const bool ok0 = lane < nq, ok1 = lane + 64 < nq;
    const int h0 = ok0 ? sqh[lane] : 0, w0 = ok0 ? sqw[lane] : 0;
    const int h1 = ok1 ? sqh[lane + 64] : 0, w1 = ok1 ? sqw[lane + 64] : 0;
    const int *T0 = sT + lane * F;
    const int *T1 = sT + (lane + 64) * F;
    for (int c = wave; c < ncand; c += kThreads / 64) {
        const int kb = scand[c];
        bool v0 = false, v1 = false;
        const int r1 = a.t.rect_off[kb + 1];
        for (int r = a.t.rect_off[kb]; r < r1; ++r) {
            const int4 rc = a.t.rects[r];
            if (ok0 && !v0) v0 = rect_dist2(rc, h0, w0) <= T0[rc.x];
            if (ok1 && !v1) v1 = rect_dist2(rc, h1, w1) <= T1[rc.x];
            if (a.vote == 1 && __any(v0 || v1)) break;
        }
        const int votes = __popcll(__ballot(v0)) + __popcll(__ballot(v1));
        if (lane == 0) sflag[kb] = votes >= a.vote ? 1 : 0;
    }
    __syncthreads();

    // 4. ascending compaction with a workgroup prefix sum
    const int chunk = (nkb + kThreads - 1) / kThreads;
    const int lo = min(nkb, tid * chunk), hi = min(nkb, lo + chunk);
    int cnt = 0;
    for (int kb = lo; kb < hi; ++kb) cnt += sflag[kb] == 1;
    sscan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int add = tid >= off ? sscan[tid - off] : 0;
        __syncthreads();
        sscan[tid] += add;
        __syncthreads();
    }
    const int64_t row = (int64_t)o * a.nqb + qb;
    int pos = sscan[tid] - cnt;
    int32_t *idx_row = a.kv_index + row * nkb;
    for (int kb = lo; kb < hi; ++kb)
        if (sflag[kb] == 1) idx_row[pos++] = kb;
    if (a.block_mask) {
        uint8_t *mrow = a.block_mask + row * nkb;
        for (int kb = tid; kb < nkb; kb += kThreads) mrow[kb] = sflag[kb] == 1;
    }
    if (tid == kThreads - 1) a.kv_count[row] = sscan[kThreads - 1];
}

}  // namespace

size_t mask_lds_bytes(int block_q, int F, int nkb) {
    const size_t ints = (size_t)block_q * F + F + 4 * (size_t)block_q + nkb + kThreads + 8;
    return ints * 4 + (size_t)nkb;
}

hipError_t launch_build_mask(const MaskArgs &a, hipStream_t s) {
    const size_t lds = mask_lds_bytes(a.block_q, a.g.F, a.nkb);
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    build_mask_kernel<<<blocks, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace tra
