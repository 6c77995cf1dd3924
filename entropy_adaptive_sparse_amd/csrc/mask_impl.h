// mask_impl.h -- device code of the mask builder: entropy -> budget -> radius -> block-sparse mask, one fused kernel
// ("Token Radius Attention for Efficient Video Generation", section 2: Insight I
// budget tau * exp(H_i) / N; Insight II radius with per-frame factor
// exp(-gamma * delta); TRA pipeline steps 2-3: a 2D disk per frame, then distance
// computation, radius comparison, block pruning and token voting fused into one
// kernel that emits a regular block-sparse mask).  Used by the standalone kernel (mask.hip)
// and as the epilogue of the fused dense+entropy+mask kernel (attention.hip).
//
// A key at squared in-frame distance d from query i, in frame f', lies in the
// query's disk iff d = 0 or ln d <= s, s = (double)H_i + lambda[f_i][f'] (one fp64
// add).  Equivalently d <= T_i(f') with the integer threshold
// T(s) = max{t : t = 0 or ln t <= s}; T is monotone in s.
//
// One workgroup per (head, q-block):
//  1. per query frame qf of the q-block (one or two frames, more for tiny frames):
//     the bounding box of its queries and Tmax[qf][f'] = T(max H + lambda[qf][f']),
//     the largest threshold any of them has toward frame f' (monotonicity of T);
//     per group of 32 queries, a "star": a query of largest entropy.
//  2. per query and frame: T_i(f') in LDS (zero without evaluation where Tmax is
//     zero).  Per target frame f': the reach window, each box grown by the integer
//     square root of its Tmax, rounded out to whole tiles; its k-blocks form one
//     contiguous range of the tile-major order (first token of the window's first
//     tile to the last token of its last tile).  No k-block outside the ranges can
//     hold a key of any disk, so only the ranges are visited, in ascending order.
//  3. the visited k-blocks, in chunks of up to 256 (one per thread).  A k-block is
//     a union of axis-aligned rectangles (host table).  A rectangle is
//       - accepted outright (vote threshold 1) when a star reaches it, with the
//         star's own threshold;
//       - dropped when it lies beyond Tmax from its frame's box (the box distance
//         bounds every query's distance from below);
//       - otherwise listed in LDS for the exact test: one wavefront per listed
//         rectangle, one lane per query (two for 128-query blocks); the squared
//         distance from a query to a rectangle is exact because the nearest lattice
//         point is the clamped query position.  Hits are ORed into the k-block's
//         per-query vote mask, so a query that reaches several rectangles of a
//         block votes once.
//  4. the chunk's retained k-blocks are appended to the ascending index list with
//     a ballot prefix sum; then the count (and the optional byte mask).
#pragma once

#include "tra_internal.h"

#include <climits>

namespace tra {
namespace maskdev {


constexpr int kThreads = kMaskThreads;
constexpr int kWaves = kThreads / 64;

typedef short short2_t __attribute__((ext_vector_type(2)));

// Squared distance between two axis-aligned boxes [alo, ahi] and [blo, bhi] of the
// lattice, each corner packed as (row | column << 16); a point is a box with equal
// corners.  Per axis the gap is max(0, a0 - b1, b0 - a1); both gaps at once in
// packed 16-bit lanes, then one 2-term dot product (sums below 2^31 for H, W < 2^15).
__device__ inline int box_dist2(int alo, int ahi, int blo, int bhi) {
    const short2_t a0 = __builtin_bit_cast(short2_t, alo), a1 = __builtin_bit_cast(short2_t, ahi);
    const short2_t b0 = __builtin_bit_cast(short2_t, blo), b1 = __builtin_bit_cast(short2_t, bhi);
    const short2_t zero = {0, 0};
    const short2_t gap = __builtin_elementwise_max(__builtin_elementwise_max(a0 - b1, b0 - a1), zero);
    return __builtin_amdgcn_sdot2(gap, gap, 0, false);
}

// T(s) = max{t <= tmax : t = 0 or lnT[t] <= s}, lnT[t] = ln t built on the host.
// Fast path: e = exp((float)s) is within a relative 3e-6 of e^s (one rounding of s
// to float, one of the exponent's argument, the exp unit's ulp), so when the
// interval e -/+ (1e-5 e + 1e-3) holds no integer, floor(e^s) is its floor and no
// rounded table entry can disagree with it (that would need e^s within a relative
// 1e-15 of an integer).  Otherwise the table decides.
__device__ inline int threshold_of(double s, const MaskTables &t) {
    if (!(s >= 0.0) || t.tmax == 0) return 0;  // s < ln 1 (or NaN): only distance 0
    if (s >= t.lnTmax) return t.tmax;          // the whole frame
    const float e = __expf((float)s);
    const float m = e * 1.0e-5f + 1.0e-3f;
    const int lo = (int)(e - m), hi = (int)(e + m);
    if (lo == hi) return lo;
    int k = max(1, min(hi, t.tmax));
    while (k < t.tmax && t.lnT[k + 1] <= s) ++k;
    while (k > 1 && t.lnT[k] > s) --k;
    return k;
}

// Order-preserving map of a non-NaN float onto unsigned ints (0 is below every key).
__device__ inline unsigned float_key(float x) {
    const unsigned b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float key_float(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline int isqrt(int v) {
    int r = (int)sqrtf((float)v);
    while (r > 0 && r * r > v) --r;
    while ((r + 1) * (r + 1) <= v) ++r;
    return r;
}

// LDS view of one workgroup's state.  Contiguous (SPLIT = false): one dynamic LDS block.
// Split (SPLIT = true): four 16 KB buffers that already exist (the attention kernel's K and V
// tiles, free once its loop is done): the exact-test list and vote masks in the first, the
// per-query thresholds of frames [0, kMaskSplitFrames) in the second and of the following
// frames in the third, everything else in the fourth.
template <int BQ, bool SPLIT>
struct MaskLds {
    static constexpr int NG = BQ / 32;                    // star groups
    static constexpr int F1 = SPLIT ? 16384 / (4 * BQ) : 0; // frames per threshold buffer
    int4 *ent;                // [kMaskEntryCap] rectangles listed for the exact test
    unsigned long long *vote; // [kThreads][2] per-query vote mask of each k-block of the chunk
    unsigned long long *gkey; // [NG] (entropy key << 32 | query) of each group's star
    double *lam;              // [QF][F] lambda rows of the q-block's frames
    int *T, *T2;              // per-query thresholds, frame-major rows of BQ (-1: no query)
    int *Tm;                  // [QF][F] largest threshold of each query frame
    int *qp, *qf;             // [BQ] packed position, frame
    float *H;                 // [BQ]
    int *box;                 // [QF][4] hmin hmax wmin wmax
    int *boxp;                // [QF][2] packed corners
    unsigned *Hk;             // [QF] largest entropy key
    int *rlo, *rhi;           // [F] k-block range of each target frame
    int *rfirst;              // [F] its first k-block not visited in an earlier range
    int *rstart;              // [F + 1] first visit index of each range
    int *star;                // [NG] query index of each star, -1 if none
    int *starp;               // [NG] its packed position
    int *wt;                  // [kWaves]
    int *n;                   // listed rectangles
    __device__ int *Trow(int f) const {
        if constexpr (SPLIT) return f < F1 ? T + f * BQ : T2 + (f - F1) * BQ;
        return T + f * BQ;
    }
    __device__ void rest(void *p, int F, int QF) {
        gkey = (unsigned long long *)p;
        lam = (double *)(gkey + NG);
        Tm = (int *)(lam + QF * F);
        qp = Tm + QF * F;
        qf = qp + BQ;
        H = (float *)(qf + BQ);
        box = (int *)(H + BQ);
        boxp = box + 4 * QF;
        Hk = (unsigned *)(boxp + 2 * QF);
        rlo = (int *)(Hk + QF);
        rhi = rlo + F;
        rfirst = rhi + F;
        rstart = rfirst + F;
        star = rstart + F + 1;
        starp = star + NG;
        wt = starp + NG;
        n = wt + kWaves;
    }
    // contiguous
    __device__ MaskLds(void *base, int F, int QF) {
        ent = (int4 *)base;
        vote = (unsigned long long *)(ent + kMaskEntryCap);
        T = (int *)(vote + 2 * kThreads);
        T2 = T;
        rest(T + F * BQ, F, QF);
    }
    // split over four 16 KB buffers
    __device__ MaskLds(void *b0, void *b1, void *b2, void *b3, int F, int QF) {
        ent = (int4 *)b0;
        vote = (unsigned long long *)(ent + kMaskEntryCap);
        T = (int *)b1;
        T2 = (int *)b2;
        rest(b3, F, QF);
    }
};

// Star test of one rectangle of frame f (vote threshold 1): some star reaches it.
template <int BQ, bool SPLIT>
__device__ inline bool star_hit(const MaskLds<BQ, SPLIT> &L, int f, int lo, int hi) {
    bool hit = false;
#pragma unroll
    for (int g = 0; g < MaskLds<BQ, SPLIT>::NG; ++g) {
        const int i = L.star[g];
        if (i >= 0) hit |= box_dist2(lo, hi, L.starp[g], L.starp[g]) <= L.Trow(f)[i];
    }
    return hit;
}

// Box test of one rectangle of frame f: some query frame's box is within its Tmax.
template <int BQ, bool SPLIT>
__device__ inline bool box_reach(const MaskLds<BQ, SPLIT> &L, int F, int nqf, int f, int lo, int hi) {
    bool h = false;
    for (int q = 0; q < nqf; ++q) h |= box_dist2(lo, hi, L.boxp[2 * q], L.boxp[2 * q + 1]) <= L.Tm[q * F + f];
    return h;
}

// Classify a k-block that is not the diagonal one from its RR rectangle slots (RR
// known at compile time; RR = 0: a.t.rmax slots read one at a time): 1 = kept by a
// star, 2 = rectangles listed for the exact test, 0 = out of reach.
template <int BQ, int RR, bool SPLIT>
__device__ inline int classify(const MaskArgs &a, const MaskLds<BQ, SPLIT> &L, int F, int nqf, int kb, int kl) {
    const bool sure = a.vote == 1;
    if constexpr (RR > 0) {
        int4 sl[RR];
#pragma unroll
        for (int r = 0; r < RR; ++r) sl[r] = a.t.rects[(int64_t)kb * RR + r];
        if (sure) {
            bool hit = false;
#pragma unroll
            for (int r = 0; r < RR; ++r)
                if (sl[r].w >= 0) hit |= star_hit<BQ, SPLIT>(L, sl[r].x, sl[r].y, sl[r].z);
            if (hit) return 1;
        }
        unsigned reach = 0;
#pragma unroll
        for (int r = 0; r < RR; ++r)
            if (sl[r].w >= 0 && box_reach<BQ, SPLIT>(L, F, nqf, sl[r].x, sl[r].y, sl[r].z)) reach |= 1u << r;
        if (!reach) return 0;
        int e = atomicAdd(L.n, __popc(reach));
#pragma unroll
        for (int r = 0; r < RR; ++r)
            if (reach >> r & 1u) L.ent[e++] = make_int4(kl | (sl[r].x << 16), sl[r].y, sl[r].z, sl[r].w);
        return 2;
    } else {
        const int4 *sl = a.t.rects + (int64_t)kb * a.t.rmax;
        const int rmax = a.t.rmax;
        if (sure) {
            for (int r = 0; r < rmax; ++r) {
                const int4 rc = sl[r];
                if (rc.w >= 0 && star_hit<BQ, SPLIT>(L, rc.x, rc.y, rc.z)) return 1;
            }
        }
        int cnt = 0;
        for (int r = 0; r < rmax; ++r) {
            const int4 rc = sl[r];
            cnt += rc.w >= 0 && box_reach<BQ, SPLIT>(L, F, nqf, rc.x, rc.y, rc.z);
        }
        if (cnt == 0) return 0;
        int e = atomicAdd(L.n, cnt);
        for (int r = 0; r < rmax; ++r) {
            const int4 rc = sl[r];
            if (rc.w >= 0 && box_reach<BQ, SPLIT>(L, F, nqf, rc.x, rc.y, rc.z))
                L.ent[e++] = make_int4(kl | (rc.x << 16), rc.y, rc.z, rc.w);
        }
        return 2;
    }
}

// Two mask rows built at once by one workgroup (the 8-wavefront warm-up kernel): each half
// of kThreads threads has its own q-block and LDS state, and both halves execute the same
// barriers -- the chunk loop runs to the larger of the two halves' visit counts, shared
// through m, and a half without a q-block (past the last one) only takes part in the
// barriers.  m = null: one row per workgroup.
struct MaskPair {
    int *m;    // [2] in LDS: visit count of each half
    int half;  // this thread's half
};

// The mask row of q-block qb of head o, by kThreads threads (tid = 0 .. kThreads - 1).
// FUSED: the q-block's entropies are already in L.H (the caller computed them); otherwise
// they are read from a.ent.  L.H must not be written between the caller's fill and this
// call.  active = false: no q-block, barriers only (pair mode).
template <int BQ, int RR, bool SPLIT, bool FUSED>
__device__ inline void mask_qblock(const MaskArgs &a, const MaskLds<BQ, SPLIT> &L, int o, int qb, int tid, bool active,
                                   MaskPair pair) {
    static_assert(BQ == 64 || BQ == 128, "one or two queries per lane");
    constexpr int NG = MaskLds<BQ, SPLIT>::NG;
    const TileGeom &g = a.g;
    const int F = g.F, nkb = a.nkb, N = g.N, QF = a.nqf_max, C = a.chunk;

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q0 = qb * BQ;
    const int nq = active ? min(BQ, N - q0) : 0;
    const int fa = active ? q0 / g.HW : 0;
    const int nqf = active ? (q0 + nq - 1) / g.HW - fa + 1 : 0;
    const float *ent = a.ent + (int64_t)o * N;
    const int64_t row = active ? (int64_t)o * a.nqb + qb : 0;
    int32_t *idx_row = a.kv_index + row * nkb;
    uint8_t *mrow = (active && a.block_mask) ? a.block_mask + row * nkb : nullptr;

    if (active) {
        for (int i = tid; i < QF; i += kThreads) {
            L.box[4 * i + 0] = INT_MAX; L.box[4 * i + 1] = INT_MIN;
            L.box[4 * i + 2] = INT_MAX; L.box[4 * i + 3] = INT_MIN;
            L.Hk[i] = 0u;
        }
        if (tid < NG) L.gkey[tid] = 0ull;
        for (int idx = tid; idx < nqf * F; idx += kThreads) L.lam[idx] = a.t.lam[fa * F + idx];
        if (mrow)
            for (int kb = tid; kb < nkb; kb += kThreads) mrow[kb] = 0;
    }
    if (tid == 0) *L.n = 0;
    __syncthreads();

    // query positions, entropies, per-frame boxes, largest entropies and stars
    for (int i = tid; i < nq; i += kThreads) {
        int f, y, x;
        tile_major_coords(q0 + i, g, f, y, x);
        const float h = FUSED ? L.H[i] : ent[q0 + i];
        L.qp[i] = y | (x << 16);
        L.qf[i] = f;
        if (!FUSED) L.H[i] = h;
        const int qf = f - fa;
        atomicMin(&L.box[4 * qf + 0], y); atomicMax(&L.box[4 * qf + 1], y);
        atomicMin(&L.box[4 * qf + 2], x); atomicMax(&L.box[4 * qf + 3], x);
        if (h == h) {
            const unsigned k = float_key(h);
            atomicMax(&L.Hk[qf], k);
            atomicMax(&L.gkey[i >> 5], ((unsigned long long)k << 32) | (unsigned)i);
        }
    }
    __syncthreads();

    // 1. frame thresholds Tmax[qf][f'], packed boxes, stars
    if (active) {
        for (int idx = tid; idx < nqf * F; idx += kThreads) {
            const int qf = idx / F;
            const unsigned k = L.Hk[qf];
            const double s = k ? (double)key_float(k) + L.lam[idx] : -INFINITY;
            L.Tm[idx] = threshold_of(s, a.t);
        }
        for (int qf = tid; qf < nqf; qf += kThreads) {
            const int *b = L.box + 4 * qf;
            L.boxp[2 * qf] = b[0] | (b[2] << 16);
            L.boxp[2 * qf + 1] = b[1] | (b[3] << 16);
        }
        if (tid < NG) {
            const unsigned long long k = L.gkey[tid];
            const int i = k ? (int)(unsigned)k : -1;
            L.star[tid] = i;
            L.starp[tid] = i >= 0 ? L.qp[i] : 0;
        }
    }
    __syncthreads();

    if (active) {
        // 2. per-query thresholds, frame-major so that a wavefront reads one frame's row
        //    (-1 marks lanes past the end of a ragged q-block: never a hit) ...
        for (int idx = tid; idx < F * BQ; idx += kThreads) {
            const int fp = idx / BQ;
            const int i = idx - fp * BQ;
            int T = -1;
            if (i < nq) {
                const int qf = L.qf[i] - fa;
                T = 0;
                if (L.Tm[qf * F + fp] > 0) T = threshold_of((double)L.H[i] + L.lam[qf * F + fp], a.t);
            }
            L.Trow(fp)[i] = T;
        }
        // ... and the k-block range of each target frame's reach window
        for (int fp = tid; fp < F; fp += kThreads) {
            int y0 = INT_MAX, y1 = INT_MIN, x0 = INT_MAX, x1 = INT_MIN;
            for (int qf = 0; qf < nqf; ++qf) {
                const int r = isqrt(L.Tm[qf * F + fp]);
                const int *b = L.box + 4 * qf;
                y0 = min(y0, b[0] - r); y1 = max(y1, b[1] + r);
                x0 = min(x0, b[2] - r); x1 = max(x1, b[3] + r);
            }
            const int ty0 = max(0, y0) / g.th, ty1 = min(g.H - 1, y1) / g.th;
            const int tx0 = max(0, x0) / g.tw, tx1 = min(g.W - 1, x1) / g.tw;
            const int ht0 = min(g.th, g.H - ty0 * g.th), ht1 = min(g.th, g.H - ty1 * g.th);
            const int wt1 = min(g.tw, g.W - tx1 * g.tw);
            const int first = fp * g.HW + ty0 * g.th * g.W + tx0 * g.tw * ht0;
            const int last = fp * g.HW + ty1 * g.th * g.W + tx1 * g.tw * ht1 + ht1 * wt1 - 1;
            L.rlo[fp] = first / a.block_k;
            L.rhi[fp] = last / a.block_k;
        }
    }
    __syncthreads();

    // ranges in ascending order: a k-block shared by two frames' ranges is visited
    // once (in the earlier one); each frame sums the visits of the frames before it
    if (active) {
        for (int fp = tid; fp <= F; fp += kThreads) {
            int pm = -1, acc = 0;
            for (int j = 0; j < fp; ++j) {
                const int hi = L.rhi[j];
                acc += max(0, hi - max(L.rlo[j], pm + 1) + 1);
                pm = max(pm, hi);
            }
            L.rstart[fp] = acc;
            if (fp < F) L.rfirst[fp] = max(L.rlo[fp], pm + 1);
        }
    }
    __syncthreads();

    const int M = active ? L.rstart[F] : 0;
    int Mloop = M;  // chunks to run: this row's, or the larger of the pair's
    if (pair.m) {
        if (tid == 0) pair.m[pair.half] = M;
        __syncthreads();
        Mloop = max(pair.m[0], pair.m[1]);
    }
    const int qp0 = active ? L.qp[min(lane, nq - 1)] : 0;
    const int qp1 = (active && BQ == 128) ? L.qp[min(lane + 64, nq - 1)] : 0;
    int run = 0;

    for (int base = 0; base < Mloop; base += C) {
        // 3a. visit index -> k-block (binary search over the frame ranges); classify
        const int v = base + tid;
        const bool mine = tid < C && v < M;
        int kb = 0, flag = 0;  // flag: 0 drop, 1 keep, 2 exact test pending
        if (mine) {
            int lo = 0, hi = F - 1;  // last frame whose range starts at or before v
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (L.rstart[mid] <= v) lo = mid; else hi = mid - 1;
            }
            kb = L.rfirst[lo] + (v - L.rstart[lo]);
            const int k0 = kb * a.block_k;
            const int k1 = min(N, k0 + a.block_k);
            L.vote[2 * tid] = 0ull;
            L.vote[2 * tid + 1] = 0ull;
            flag = (k0 < q0 + nq && q0 < k1) ? 1 : classify<BQ, RR, SPLIT>(a, L, F, nqf, kb, tid);
        }
        __syncthreads();

        // 3b. exact test, two listed rectangles per wavefront per step, one lane per query
        const int ne = __builtin_amdgcn_readfirstlane(*L.n);
        for (int e = 2 * wave; e < ne; e += 2 * kWaves) {
            const int4 A = L.ent[e];
            const int4 B = L.ent[min(e + 1, ne - 1)];
            const int ax = __builtin_amdgcn_readfirstlane(A.x), ay = __builtin_amdgcn_readfirstlane(A.y),
                      az = __builtin_amdgcn_readfirstlane(A.z);
            const int bx = __builtin_amdgcn_readfirstlane(B.x), by = __builtin_amdgcn_readfirstlane(B.y),
                      bz = __builtin_amdgcn_readfirstlane(B.z);
            const int *TA = L.Trow(ax >> 16) + lane;
            const int *TB = L.Trow(bx >> 16) + lane;
            const unsigned long long a0 = __ballot(box_dist2(ay, az, qp0, qp0) <= TA[0]);
            const unsigned long long b0 = __ballot(box_dist2(by, bz, qp0, qp0) <= TB[0]);
            unsigned long long a1 = 0ull, b1 = 0ull;
            if (BQ == 128) {
                a1 = __ballot(box_dist2(ay, az, qp1, qp1) <= TA[64]);
                b1 = __ballot(box_dist2(by, bz, qp1, qp1) <= TB[64]);
            }
            if (lane == 0) {
                if (a0 | a1) {
                    atomicOr(&L.vote[2 * (ax & 0xffff)], a0);
                    if (BQ == 128) atomicOr(&L.vote[2 * (ax & 0xffff) + 1], a1);
                }
                if (b0 | b1) {
                    atomicOr(&L.vote[2 * (bx & 0xffff)], b0);
                    if (BQ == 128) atomicOr(&L.vote[2 * (bx & 0xffff) + 1], b1);
                }
            }
        }
        __syncthreads();

        // 4. votes -> kept flags -> ascending compaction of this chunk
        bool keep = flag == 1;
        if (flag == 2) keep = __popcll(L.vote[2 * tid]) + __popcll(L.vote[2 * tid + 1]) >= a.vote;
        const unsigned long long bal = __ballot(keep);
        if (lane == 0) L.wt[wave] = (int)__popcll(bal);
        if (tid == 0) *L.n = 0;
        __syncthreads();
        int pos = run + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
        for (int w = 0; w < wave; ++w) pos += L.wt[w];
        if (keep) {
            idx_row[pos] = kb;
            if (mrow) mrow[kb] = 1;
        }
        for (int w = 0; w < kWaves; ++w) run += L.wt[w];
    }
    if (active && tid == 0) a.kv_count[row] = run;
}

}  // namespace maskdev
}  // namespace tra
