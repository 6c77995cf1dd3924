// mask.hip -- the standalone mask kernel (entropy -> budget -> radius -> block-sparse
// mask; "Token Radius Attention for Efficient Video Generation", section 2: Insight I,
// Insight II, TRA pipeline steps 2-3), one workgroup per (head, q-block); the device code
// and its description are in mask_impl.h.
#include "mask_impl.h"

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
