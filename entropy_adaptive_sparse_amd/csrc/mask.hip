// mask.hip -- the standalone mask kernel (entropy -> budget -> radius -> block-sparse
// mask; "Token Radius Attention for Efficient Video Generation", section 2: Insight I,
// Insight II, TRA pipeline steps 2-3), one workgroup per (head, q-block); the device code
// and its description are in mask_impl.h.
#include "mask_impl.h"

#include <algorithm>

namespace tra {

namespace {

using namespace maskdev;

template <int BQ, int RR>
__global__ __launch_bounds__(kThreads) void build_mask_kernel(MaskArgs a) {
    extern __shared__ int4 smem4[];
    const MaskLds<BQ, false> L(smem4, a.g.F, a.nqf_max);
    const int o = blockIdx.x / a.nqb;
    mask_qblock<BQ, RR, false, false>(a, L, o, blockIdx.x - o * a.nqb, threadIdx.x, true, MaskPair{nullptr, 0});
}

}  // namespace

int mask_frames_per_qblock(int block_q, int HW, int F) {
    return std::min(F, (block_q - 1) / HW + 2);
}

// bytes of everything but the list, the vote masks and the per-query thresholds
static size_t mask_rest_bytes(int block_q, int F, int HW) {
    const int qf = mask_frames_per_qblock(block_q, HW, F);
    const int ng = block_q / 32;
    const size_t ints = (size_t)qf * F + 3 * (size_t)block_q + 7 * (size_t)qf + 4 * (size_t)F + 1 + 2 * (size_t)ng +
                        maskdev::kWaves + 1;
    return ng * sizeof(unsigned long long) + (size_t)qf * F * sizeof(double) + ints * 4;
}

size_t mask_lds_bytes(int block_q, int F, int HW) {
    return (size_t)kMaskEntryCap * sizeof(int4) + 2 * maskdev::kThreads * sizeof(unsigned long long) +
           (size_t)F * block_q * 4 + mask_rest_bytes(block_q, F, HW);
}

bool mask_fits_split(int block_q, int F, int HW) {
    const int f1 = 16384 / (4 * block_q);
    return block_q == 128 && F <= 2 * f1 && mask_rest_bytes(block_q, F, HW) <= 16384 &&
           (size_t)kMaskEntryCap * sizeof(int4) + 2 * maskdev::kThreads * sizeof(unsigned long long) <= 16384;
}

template <int BQ>
static hipError_t launch_bq(const MaskArgs &a, size_t lds, unsigned blocks, hipStream_t s) {
    switch (a.t.rmax) {
        case 1: build_mask_kernel<BQ, 1><<<blocks, kThreads, lds, s>>>(a); break;
        case 2: build_mask_kernel<BQ, 2><<<blocks, kThreads, lds, s>>>(a); break;
        case 3: build_mask_kernel<BQ, 3><<<blocks, kThreads, lds, s>>>(a); break;
        case 4: build_mask_kernel<BQ, 4><<<blocks, kThreads, lds, s>>>(a); break;
        default: build_mask_kernel<BQ, 0><<<blocks, kThreads, lds, s>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_build_mask(const MaskArgs &a, hipStream_t s) {
    const size_t lds = mask_lds_bytes(a.block_q, a.g.F, a.g.HW);
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    return a.block_q == 128 ? launch_bq<128>(a, lds, blocks, s) : launch_bq<64>(a, lds, blocks, s);
}

}  // namespace tra
