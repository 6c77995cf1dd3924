// mask_sizes.cpp -- host-side sizes of the mask builder's on-chip state (LDS bytes, frames
// per q-block), shared by the argument checks of the C ABI and the kernel launches.  The
// layout is the one mask_impl.h (MaskLds) lays out.
#include "tra_internal.h"

#include <algorithm>

namespace tra {

int mask_frames_per_qblock(int block_q, int HW, int F) {
    return std::min(F, (block_q - 1) / HW + 2);
}

// bytes of everything but the list, the vote masks and the per-query thresholds
static size_t mask_rest_bytes(int block_q, int F, int HW) {
    const int qf = mask_frames_per_qblock(block_q, HW, F);
    const int ng = block_q / 32;
    const size_t ints = (size_t)qf * F + 3 * (size_t)block_q + 7 * (size_t)qf + 4 * (size_t)F + 1 + 2 * (size_t)ng +
                        (kMaskThreads / 64) + 1;
    return ng * sizeof(unsigned long long) + (size_t)qf * F * sizeof(double) + ints * 4;
}

size_t mask_lds_bytes(int block_q, int F, int HW) {
    return (size_t)kMaskEntryCap * sizeof(int4) + 2 * kMaskThreads * sizeof(unsigned long long) +
           (size_t)F * block_q * 4 + mask_rest_bytes(block_q, F, HW);
}

bool mask_fits_split(int block_q, int F, int HW) {
    const int f1 = 16384 / (4 * block_q);
    return block_q == 128 && F <= 2 * f1 && mask_rest_bytes(block_q, F, HW) <= 16384 &&
           (size_t)kMaskEntryCap * sizeof(int4) + 2 * kMaskThreads * sizeof(unsigned long long) <= 16384;
}

}  // namespace tra
