// mask1d.hip -- the 1D-distance variant of the mask ("Token Radius Attention for Efficient Video
// Generation", section 4, ablation study: the radius mask replaced by a 1D distance), built into
// the same regular block-sparse format as the disk mask.
//
// Query i keeps key j iff d = |n_i - n_j| is 0 or ln d <= (double)H_i + mu, n the natural raster
// index (f*H + h)*W + w and mu = ln tau - ln 2 (fp64, host): the window 2 d <= tau exp(H_i) of
// the budget of Insight I around the query in the flattened sequence.  With the integer threshold
// T_i = max{t : t = 0 or ln t <= s_i} (the disk builder's threshold_of, on a table of ln t for
// t < N), the window is the natural index interval [n_i - T_i, n_i + T_i].
//
// One workgroup per (head, q-block), the k-blocks in chunks of 256 (one per thread):
//  1. per query: natural index, threshold, window; the q-block's hull (union bound of windows);
//  2. per chunk: candidates = k-blocks whose natural-index hull meets the q-block's hull, and the
//     diagonal ones (no key of any other k-block lies in any window), compacted in order;
//  3. one wavefront per candidate: lane l tests queries l and l + 64 against the k-block's
//     rectangles exactly (a rectangle row is one run of natural indices) and the ballots count the
//     votes; kept iff votes >= threshold or diagonal;
//  4. the kept candidates are appended to the ascending index list; the count (and byte mask).
#include "mask_impl.h"
#include "tra_internal.h"

namespace tra {

namespace {

constexpr int kT = 256;  // threads per workgroup = k-blocks per chunk

// whether natural-index window [a, b] (a <= b) meets rectangle rc {f, y0 | x0 << 16, y1 | x1 << 16,
// f or -1}: some row y of [y0, y1] whose run [(f H + y) W + x0, (f H + y) W + x1] meets [a, b]
__device__ inline bool window_meets(int a, int b, int4 rc, int H, int W) {
    if (rc.w < 0) return false;  // unused slot
    const int y0 = rc.y & 0xffff, x0 = rc.y >> 16, y1 = rc.z & 0xffff, x1 = rc.z >> 16;
    const int base = rc.x * H;
    // run start <= b: y <= floor((b - x0) / W) - base; run end >= a: y >= ceil((a - x1) / W) - base
    // (b - x0 and a - x1 are at least -(W - 1): the shifted divisions below are on non-negative values)
    const int ylo = max(y0, (a - x1 + W - 1) / W - base);
    const int yhi = min(y1, (b - x0 + W) / W - 1 - base);
    return ylo <= yhi;
}

template <int BQ>
__global__ __launch_bounds__(kT) void build_mask_1d_kernel(WindowArgs a) {
    __shared__ int qlo[BQ], qhi[BQ];  // query windows (empty: lo > hi)
    __shared__ int hull[2];
    __shared__ int list[kT];          // candidates of the chunk, ascending
    __shared__ int kept[kT];          // 1 = candidate kept (same slots as list)
    __shared__ int wcount[kT / 64];
    __shared__ int base_out;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int o = blockIdx.x / a.nqb;
    const int qb = blockIdx.x - o * a.nqb;
    const int N = a.g.N;
    const int q0 = qb * BQ, q1 = min(N, q0 + BQ);
    const int64_t row = (int64_t)o * a.nqb + qb;

    if (tid == 0) {
        hull[0] = INT_MAX;
        hull[1] = -1;
        base_out = 0;
    }
    __syncthreads();
    // 1. windows
    if (tid < BQ) {
        int lo = 1, hi = 0;
        const int p = q0 + tid;
        if (p < N) {
            const int n = tile_major_to_natural(p, a.g);
            MaskTables mt{};
            mt.lnT = a.t.lnT;
            mt.tmax = N - 1;
            mt.lnTmax = a.t.lnTmax;
            const double s = (double)a.ent[(int64_t)o * N + p] + a.t.mu;
            const int T = maskdev::threshold_of(s, mt);
            lo = max(0, n - T);
            hi = min(N - 1, n + T);
            atomicMin(&hull[0], lo);
            atomicMax(&hull[1], hi);
        }
        qlo[tid] = lo;
        qhi[tid] = hi;
    }
    __syncthreads();
    const int hlo = hull[0], hhi = hull[1];
    const int H = a.g.H, W = a.g.W, rmax = a.t.rmax;

    for (int c0 = 0; c0 < a.nkb; c0 += kT) {
        // 2. candidates of the chunk, compacted in ascending order
        const int kb = c0 + tid;
        bool cand = false, diag = false;
        if (kb < a.nkb) {
            const int k0 = kb * a.block_k, k1 = min(N, k0 + a.block_k);
            diag = k0 < q1 && q0 < k1;
            const int2 h = a.t.hull[kb];
            cand = diag || (h.x <= hhi && hlo <= h.y);
        }
        const unsigned long long bal = __ballot(cand);
        const int rank = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (lane == 0) wcount[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, ncand = 0;
        for (int w = 0; w < kT / 64; ++w) {
            before += w < wave ? wcount[w] : 0;
            ncand += wcount[w];
        }
        if (cand) list[before + rank] = kb;
        __syncthreads();
        // 3. exact test, one wavefront per candidate
        for (int i = wave; i < ncand; i += kT / 64) {
            const int kbi = list[i];
            bool h0 = false, h1 = false;
            const int a0 = qlo[lane], b0 = qhi[lane];
            const int a1 = BQ > 64 ? qlo[lane + 64] : 1, b1 = BQ > 64 ? qhi[lane + 64] : 0;
            for (int r = 0; r < rmax; ++r) {
                const int4 rc = a.t.rects[(int64_t)kbi * rmax + r];
                if (a0 <= b0) h0 |= window_meets(a0, b0, rc, H, W);
                if (a1 <= b1) h1 |= window_meets(a1, b1, rc, H, W);
            }
            const int votes = __popcll(__ballot(h0)) + __popcll(__ballot(h1));
            if (lane == 0) {
                const int k0 = kbi * a.block_k, k1 = min(N, k0 + a.block_k);
                kept[i] = (votes >= a.vote || (k0 < q1 && q0 < k1)) ? 1 : 0;
            }
        }
        __syncthreads();
        // 4. kept candidates appended in order; the byte mask of the chunk
        const bool keep = tid < ncand && kept[tid];
        const unsigned long long kb2 = __ballot(keep);
        const int krank = __popcll(kb2 & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        __syncthreads();  // every wavefront has read wcount and kept
        if (lane == 0) wcount[wave] = __popcll(kb2);
        __syncthreads();
        int kbefore = 0, nkept = 0;
        for (int w = 0; w < kT / 64; ++w) {
            kbefore += w < wave ? wcount[w] : 0;
            nkept += wcount[w];
        }
        const int out0 = base_out;
        if (keep) a.kv_index[row * a.nkb + out0 + kbefore + krank] = list[tid];
        if (a.block_mask && kb < a.nkb) a.block_mask[row * a.nkb + kb] = 0;
        __syncthreads();
        if (a.block_mask && keep) a.block_mask[row * a.nkb + list[tid]] = 1;
        if (tid == 0) base_out = out0 + nkept;
        __syncthreads();
    }
    if (tid == 0) a.kv_count[row] = base_out;
}

}  // namespace

hipError_t launch_build_mask_1d(const WindowArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    if (a.block_q == 128)
        build_mask_1d_kernel<128><<<blocks, kT, 0, s>>>(a);
    else
        build_mask_1d_kernel<64><<<blocks, kT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace tra
