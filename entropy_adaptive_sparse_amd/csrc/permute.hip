// permute.hip -- tile-major permutation of token rows ("Token Radius Attention for
// Efficient Video Generation", section 2, TRA pipeline step 3: tokens reordered
// tile-major so that spatial neighbours are contiguous in the sequence).
//
// Pure HBM-bound data movement: every row is read once and written once.  A wave
// owns 64 consecutive destination rows (permute) or source rows (unpermute); each
// lane evaluates the closed-form tile-major map for one row, and the wave then
// streams the 64 rows with all lanes on consecutive 16-byte units of a row, so
// every load and store instruction covers whole contiguous row segments.
#include "tra_internal.h"

namespace tra {

namespace {

// 16-byte unit as a native vector (the nontemporal builtins take no struct types)
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Units in flight per lane before the stores: 2 for the permute (scattered reads), 4 for the
// unpermute (scattered writes), the faster of 2, 4, 6 and 8 for each (measured at 720p).
// Loads and stores are nontemporal: every byte is touched once, so it need not stay in the
// caches (+7-8% over plain accesses).
template <typename U, int UPR, int DIR>
__global__ __launch_bounds__(256) void permute_kernel(const U *__restrict__ src, U *__restrict__ dst,
                                                      int64_t total_rows, int N, TileGeom g, int upr_rt) {
    constexpr int kBatch = DIR == 0 ? 2 : 4;
    const int dir = DIR;
    const int upr = UPR > 0 ? UPR : upr_rt;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t base = wave * 64; base < total_rows; base += nwaves * 64) {
        const int64_t row = base + lane;
        int64_t nat_row = 0;
        if (row < total_rows) {
            const int o = (int)(row / N);
            const int p = (int)(row - (int64_t)o * N);
            nat_row = (int64_t)o * N + tile_major_to_natural(p, g);
        }
        const int rows_here = (int)min<int64_t>(64, total_rows - base);
        const int units = rows_here * upr;
        for (int idx0 = 0; idx0 < units; idx0 += 64 * kBatch) {
            U val[kBatch];
            int64_t daddr[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int idx = idx0 + b * 64 + lane;
                const int rr = idx / upr;
                const int u = idx - rr * upr;
                const int64_t nat = __shfl(nat_row, rr < 64 ? rr : 0);
                const int64_t tm = base + rr;
                daddr[b] = -1;
                if (idx < units) {
                    const int64_t s_row = dir == 0 ? nat : tm;
                    const int64_t d_row = dir == 0 ? tm : nat;
                    val[b] = __builtin_nontemporal_load(&src[s_row * upr + u]);
                    daddr[b] = d_row * upr + u;
                }
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (daddr[b] >= 0) __builtin_nontemporal_store(val[b], &dst[daddr[b]]);
        }
    }
}

template <typename U, int DIR>
hipError_t launch_dir(const U *sp, U *dp, int64_t total_rows, const TileGeom &g, int upr, unsigned blocks,
                      hipStream_t s) {
    if (upr == 16)
        permute_kernel<U, 16, DIR><<<blocks, 256, 0, s>>>(sp, dp, total_rows, g.N, g, upr);
    else if (upr == 8)
        permute_kernel<U, 8, DIR><<<blocks, 256, 0, s>>>(sp, dp, total_rows, g.N, g, upr);
    else if (upr == 32)
        permute_kernel<U, 32, DIR><<<blocks, 256, 0, s>>>(sp, dp, total_rows, g.N, g, upr);
    else if (upr == 1)
        permute_kernel<U, 1, DIR><<<blocks, 256, 0, s>>>(sp, dp, total_rows, g.N, g, upr);
    else
        permute_kernel<U, 0, DIR><<<blocks, 256, 0, s>>>(sp, dp, total_rows, g.N, g, upr);
    return hipGetLastError();
}

template <typename U>
hipError_t launch_typed(const void *src, void *dst, int outer, const TileGeom &g, int64_t row_bytes, int dir,
                        hipStream_t s) {
    const int upr = (int)(row_bytes / (int64_t)sizeof(U));
    const int64_t total_rows = (int64_t)outer * g.N;
    const int64_t waves = (total_rows + 63) / 64;
    const int64_t blocks64 = (waves + 3) / 4;
    const unsigned blocks = (unsigned)(blocks64 < (1 << 30) ? blocks64 : (1 << 30));
    const U *sp = static_cast<const U *>(src);
    U *dp = static_cast<U *>(dst);
    if (dir == 0) return launch_dir<U, 0>(sp, dp, total_rows, g, upr, blocks, s);
    return launch_dir<U, 1>(sp, dp, total_rows, g, upr, blocks, s);
}

}  // namespace

hipError_t launch_permute(const void *src, void *dst, int outer, const TileGeom &g, int64_t row_bytes, int dir,
                          hipStream_t s) {
    const uintptr_t align = (uintptr_t)src | (uintptr_t)dst;
    if (row_bytes % 16 == 0 && align % 16 == 0) return launch_typed<u32x4_t>(src, dst, outer, g, row_bytes, dir, s);
    if (row_bytes % 4 == 0 && align % 4 == 0) return launch_typed<uint32_t>(src, dst, outer, g, row_bytes, dir, s);
    if (row_bytes % 2 == 0 && align % 2 == 0) return launch_typed<uint16_t>(src, dst, outer, g, row_bytes, dir, s);
    return launch_typed<uint8_t>(src, dst, outer, g, row_bytes, dir, s);
}

}  // namespace tra
