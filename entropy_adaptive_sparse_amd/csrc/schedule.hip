// schedule.hip -- the order in which the block-sparse attention kernel's workgroups take the
// (head, q-block) rows ("Token Radius Attention for Efficient Video Generation", section 4:
// 9-19% of the interactions are kept, with per-query budgets that differ by orders of magnitude,
// so the retained k-block lists -- the work of each row -- differ in length).
//
// Two orders, both permutations of the rows o * nqb + qb:
//  - longest first (a list-scheduling order): rows sorted by kv_count, largest first, ties by
//    row.  Workgroups are dispatched in grid order as slots free up, so the shortest rows end the
//    grid and the tail is short.  Used when the grid is under two waves of resident workgroups.
//  - spatial band order: within a head, rows sorted by (row of tiles, frame, position along the
//    row of tiles) of their centre token -- runs of q-blocks that sit in the same band of the
//    frame across consecutive frames, whose lists share most of their k-blocks -- cut into runs
//    of kBandRun rows per XCD (workgroup b goes to XCD b mod 8), the runs of the 8 XCDs advancing
//    together through the heads.  Used for larger grids, where the L2 of each XCD is the issue.
#include "tra_internal.h"

namespace tra {

namespace {

__global__ void band_order_kernel(const int32_t *__restrict__ band, int nqb, int total, int32_t *__restrict__ order) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= total) return;
    const int L = xcd_runs(b, total);
    const int o = L / nqb, r = L - o * nqb;
    order[b] = o * nqb + band[r];
}

// Stable counting sort of the rows by key nkb - min(max(kv_count, 0), nkb) (largest count first),
// one workgroup: a histogram of the keys in LDS, its exclusive scan, then one wavefront places
// the rows in row order, 64 at a time, each row after the rows of equal key before it (ranks
// within a group of 64 from ballots over the key bits, so the order is deterministic).
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void lpt_order_kernel(const int32_t *__restrict__ cnt, int nkb, int total,
                                                                 int32_t *__restrict__ order) {
    extern __shared__ int hist[];  // nkb + 1 bins
    const int nb = nkb + 1;
    for (int i = threadIdx.x; i < nb; i += kSortThreads) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < total; i += kSortThreads) {
        const int key = nkb - min(max(cnt[i], 0), nkb);
        atomicAdd(&hist[key], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // exclusive scan (at most a few thousand bins, once per warm-up)
        int run = 0;
        for (int i = 0; i < nb; ++i) {
            const int c = hist[i];
            hist[i] = run;
            run += c;
        }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int kbits = 1;
        while ((1 << kbits) <= nkb) ++kbits;
        const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int base = 0; base < total; base += 64) {
            const int i = base + lane;
            const bool valid = i < total;
            const int key = valid ? nkb - min(max(cnt[i], 0), nkb) : -1;
            // lanes holding the same key: agree on every key bit (and on validity)
            unsigned long long same = __ballot(valid);
            if (!valid) same = ~same;
            for (int bit = 0; bit < kbits; ++bit) {
                const bool set = valid && ((key >> bit) & 1);
                const unsigned long long bal = __ballot(set);
                same &= set ? bal : ~bal;
            }
            const int rank = __popcll(same & below);
            const int pos = valid ? hist[key] + rank : 0;
            // every lane has read hist[key] before the first of its group advances it
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                order[pos] = i;
                if ((same & below) == 0) hist[key] += __popcll(same);  // the group's first lane
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s) {
    const int total = a.outer * a.nqb;
    if (a.lpt) {
        const size_t lds = sizeof(int) * (size_t)(a.nkb + 1);
        lpt_order_kernel<<<1, kSortThreads, lds, s>>>(a.kv_count, a.nkb, total, a.order);
    } else {
        band_order_kernel<<<(total + 255) / 256, 256, 0, s>>>(a.band, a.nqb, total, a.order);
    }
    return hipGetLastError();
}

}  // namespace tra
