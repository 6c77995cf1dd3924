// The host side of libtra.so (argument validation, the per-device table caches, the host
// table builders and the argument plumbing to the launchers) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU.  The HIP runtime calls and the kernel launchers
// are replaced by host stand-ins: device memory is host memory, and each launcher records
// its arguments.  Built and run by tests/test_sanitizers.py; prints "host sanitize ok".
#include <algorithm>
using std::max;
using std::min;

#include "../../entropy_adaptive_sparse_amd/csrc/mask_sizes.cpp"
#include "../../entropy_adaptive_sparse_amd/csrc/tra_api.cpp"

#include <cstdio>
#include <cstdlib>
#include <vector>

// ---------------------------------------------------------------- stand-ins
extern "C" {
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipMalloc(void **p, size_t n) {
    *p = std::malloc(n);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) {
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "stand-in"; }
}

namespace {
int g_launches = 0;
tra::MaskArgs g_mask;
tra::AttnArgs g_attn;
}  // namespace

namespace tra {
hipError_t launch_permute(const void *, void *, int, const TileGeom &, int64_t, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attention(const AttnArgs &a, int, int, int, bool, hipStream_t) {
    g_attn = a;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attention_natural(const AttnArgs &a, bool, hipStream_t) {
    g_attn = a;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_build_mask(const MaskArgs &m, hipStream_t) {
    g_mask = m;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_dense_mask(const AttnArgs &a, const MaskArgs &m, hipStream_t) {
    g_attn = a;
    g_mask = m;
    ++g_launches;
    return hipSuccess;
}
}  // namespace tra

#define CHECK(cond, msg)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::fprintf(stderr, "failed: %s\n", msg);    \
            return 1;                                     \
        }                                                 \
    } while (0)

int main() {
    // mask tables for the workload grids and some ragged ones (host builders run here)
    const int grids[][5] = {{21, 45, 80, 8, 8}, {33, 45, 80, 8, 8}, {21, 30, 52, 8, 8}, {3, 15, 17, 8, 8},
                            {2, 9, 7, 4, 3},    {1, 1, 1, 8, 8},    {40, 2, 3, 8, 8}};
    for (const auto &gd : grids)
        for (int bq : {64, 128})
            CHECK(tra_mask_prepare(gd[0], gd[1], gd[2], 0.03f, 0.5f, bq, 64, gd[3], gd[4]) == TRA_OK, "mask_prepare");

    // the mask call reaches its launcher with the sizes the kernel assumes
    {
        const int F = 21, H = 45, W = 80, N = F * H * W, nqb = (N + 127) / 128, nkb = (N + 63) / 64;
        std::vector<float> ent((size_t)2 * N, 5.0f);
        std::vector<int32_t> cnt((size_t)2 * nqb), idx((size_t)2 * nqb * nkb);
        CHECK(tra_build_block_mask(ent.data(), 2, F, H, W, 0.03f, 0.5f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                   (int64_t)idx.size(), nullptr, nullptr) == TRA_OK,
              "build_block_mask");
        CHECK(g_mask.nqb == nqb && g_mask.nkb == nkb && g_mask.t.rmax == 3 && g_mask.nqf_max == 2, "mask args");
        CHECK(g_mask.chunk == 256 && g_mask.t.tmax == 44 * 44 + 79 * 79, "mask chunk / tmax");
        CHECK(tra_build_block_mask(ent.data(), 2, F, H, W, 0.03f, 0.5f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                   (int64_t)idx.size() - 1, nullptr, nullptr) == TRA_ERR_CAPACITY,
              "capacity");
    }

    // natural-order calls build the map; it matches the closed form run by run
    {
        const int F = 3, H = 15, W = 20, N = F * H * W, D = 128;
        std::vector<uint16_t> q((size_t)N * D), k(q.size()), v(q.size()), o(q.size());
        std::vector<int32_t> cnt((N + 127) / 128, 1), idx((size_t)((N + 127) / 128) * ((N + 63) / 64), 0);
        CHECK(tra_block_sparse_attn_natural(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1,
                                            F, H, W, D, TRA_BF16, 0.088f, 128, 64, 8, 8, nullptr) == TRA_OK,
              "sparse natural");
        CHECK(g_attn.nat4 != nullptr, "natural map");
        tra::TileGeom g{F, H, W, 8, 8, H * W, N};
        for (int p = 0; p < N; ++p)
            CHECK(g_attn.nat4[p / 4] + p % 4 == tra::tile_major_to_natural(p, g), "natural map entry");
        CHECK(tra_dense_attn_entropy_natural(q.data(), k.data(), v.data(), o.data(), nullptr, nullptr, 1, F, 15, 18, D,
                                             TRA_BF16, 0.088f, 8, 8, nullptr) == TRA_ERR_UNSUPPORTED,
              "W not a multiple of 4");
    }

    // the fused warm-up and the plain calls, valid and invalid
    {
        const int F = 4, H = 16, W = 16, N = F * H * W, D = 128, nqb = N / 128, nkb = N / 64;
        std::vector<uint16_t> q((size_t)N * D), k(q.size()), v(q.size()), o(q.size());
        std::vector<float> ent(N), lse(N);
        std::vector<int32_t> cnt(nqb), idx((size_t)nqb * nkb);
        CHECK(tra_dense_attn_entropy_mask(q.data(), k.data(), v.data(), o.data(), ent.data(), lse.data(), 1, F, H, W, D,
                                          TRA_BF16, 0.088f, 0.03f, 0.5f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                          (int64_t)idx.size(), nullptr, nullptr) == TRA_OK,
              "fused");
        CHECK(tra_dense_attn_entropy_mask_natural(q.data(), k.data(), v.data(), o.data(), ent.data(), lse.data(), 1, F,
                                                  H, W, D, TRA_BF16, 0.088f, 0.03f, 0.5f, 128, 64, 1, 8, 8,
                                                  cnt.data(), idx.data(), (int64_t)idx.size(), nullptr,
                                                  nullptr) == TRA_OK,
              "fused natural");
        CHECK(tra_dense_attn_entropy(q.data(), k.data(), v.data(), o.data(), ent.data(), nullptr, 1, N, D, TRA_BF16,
                                     0.088f, nullptr) == TRA_OK,
              "dense");
        CHECK(tra_block_sparse_attn(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1, N, D,
                                    TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_OK,
              "sparse");
        CHECK(tra_tile_major_permute(q.data(), o.data(), 1, F, H, W, D, TRA_BF16, 8, 8, nullptr) == TRA_OK, "permute");
        CHECK(tra_block_sparse_attn(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1, N, 96,
                                    TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_ERR_UNSUPPORTED,
              "D = 96");
        CHECK(tra_dense_attn_entropy(nullptr, k.data(), v.data(), o.data(), nullptr, nullptr, 1, N, D, TRA_BF16,
                                     0.088f, nullptr) == TRA_ERR_INVALID_ARG,
              "null q");
    }
    CHECK(g_launches == 7, "launch count");
    std::printf("host sanitize ok\n");
    return 0;
}
