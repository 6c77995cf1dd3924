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
// allocations, host <-> device copies and attribute queries the library makes (none may follow
// the prepare calls on the paths they prepare)
int g_mallocs = 0, g_copies = 0, g_attrs = 0;

extern "C" {
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipMalloc(void **p, size_t n) {
    ++g_mallocs;
    *p = std::malloc(n);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) {
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
    ++g_copies;
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
    ++g_attrs;
    *v = 256;
    return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stand-in"; }
}

namespace {
int g_launches = 0;
tra::MaskArgs g_mask;
tra::AttnArgs g_attn;
tra::ScheduleArgs g_sched;
tra::WindowArgs g_win_args;
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

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t) {
    g_sched = a;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_build_mask_1d(const WindowArgs &a, hipStream_t) {
    g_win_args = a;
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_attention_fp8(const AttnArgs &a, hipStream_t) {
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

// Bounds model of the block-sparse attention kernel's tile copies.  The kernel walks a list of
// ntiles entries in steps; step j computes tile j and copies K of tile j + 2 and V of tile j + 1.
// The first sparse_fast_steps(ntiles) steps issue those copies between their products as whole
// 64-row tiles (tile-major base + 64 rows) with the list entries taken through
// sparse_full_kblock; the later steps, and the copies before the first step, go through the
// row-by-row path, which reads row min(r, N - 1) of the k-block sparse_kblock names.  Every list
// of every length below, valid or not, must keep each whole-tile copy inside [0, N) and name a
// k-block in [0, nkb) for the row-by-row path.
int check_sparse_copy_bounds() {
    unsigned rng = 12345u;
    auto next = [&rng]() {
        rng = rng * 1664525u + 1013904223u;
        return (int)(rng >> 8);
    };
    const int sizes[] = {64, 65, 100, 127, 1000, 1024, 4096 + 16, 75600};
    for (int N : sizes) {
        const int nkb = (N + 63) / 64, nfull = N / 64;
        for (int ntiles = 0; ntiles <= std::min(nkb, 40) + 3; ++ntiles) {
            const int len = std::min(ntiles, nkb);  // the kernel clamps the count into [0, nkb]
            for (int trial = 0; trial < 64; ++trial) {
                std::vector<int> list((size_t)std::max(len, 1));
                for (int i = 0; i < len; ++i) {
                    const int kind = next() % 6;
                    // valid-looking entries, the ragged k-block anywhere, negative and huge values
                    list[(size_t)i] = kind == 0 ? nkb - 1 : kind == 1 ? -(next() % 100) - 1
                                    : kind == 2 ? nkb + next() % 1000 : next() % nkb;
                }
                const int fast = tra::sparse_fast_steps(len);
                for (int j = 0; j < len; ++j) {
                    if (j < fast) {
                        // K of tile j + 2, V of tile j + 1, the entry of tile j + 3 read ahead
                        for (int t : {j + 1, j + 2, j + 3}) {
                            if (t >= len) {
                                std::fprintf(stderr, "fast step %d of %d reads past the list\n", j, len);
                                return 1;
                            }
                            const int kb = tra::sparse_full_kblock(list[(size_t)t], nfull);
                            if (kb < 0 || (int64_t)kb * 64 + 64 > N) {
                                std::fprintf(stderr, "whole-tile copy of k-block %d past N = %d\n", kb, N);
                                return 1;
                            }
                        }
                    }
                    const int kb = tra::sparse_kblock(list[(size_t)j], nkb);
                    if (kb < 0 || kb >= nkb) {
                        std::fprintf(stderr, "row-by-row copy of k-block %d outside [0, %d)\n", kb, nkb);
                        return 1;
                    }
                }
                // a valid list (ascending, distinct) never has the ragged k-block before its last entry,
                // so the whole-tile clamp leaves every entry a fast step fetches unchanged
                std::vector<int> valid;
                for (int kb = 0; kb < nkb && (int)valid.size() < len; ++kb)
                    if (next() % 3 == 0 || nkb - kb <= len - (int)valid.size()) valid.push_back(kb);
                for (int j = 0; j < fast; ++j)
                    for (int t : {j + 1, j + 2, j + 3})
                        if (t < len - 1 && tra::sparse_full_kblock(valid[(size_t)t], nfull) != valid[(size_t)t]) {
                            std::fprintf(stderr, "clamp changed a valid entry\n");
                            return 1;
                        }
            }
        }
    }
    return 0;
}

int main() {
    CHECK(check_sparse_copy_bounds() == 0, "sparse copy bounds");

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
        CHECK(tra_natural_prepare(F, H, W, 8, 8) == TRA_OK, "natural prepare (cached map)");
        CHECK(tra_natural_prepare(F, H, 18, 8, 8) == TRA_ERR_UNSUPPORTED, "natural prepare, W = 18");
        CHECK(tra_natural_prepare(2, 6, 8, 3, 4) == TRA_OK, "natural prepare, new geometry");
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
        CHECK(tra_block_sparse_attn_fp8(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), nullptr,
                                        1, N, D, 0.088f, 128, 64, nullptr) == TRA_OK && g_attn.kv_index == idx.data(),
              "sparse fp8");
        CHECK(tra_block_sparse_attn_fp8(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), nullptr,
                                        1, N, 64, 0.088f, 128, 64, nullptr) == TRA_ERR_UNSUPPORTED,
              "sparse fp8, D = 64");
        CHECK(tra_block_sparse_attn_fp8(q.data(), k.data(), v.data(), o.data(), nullptr, nullptr, idx.data(), nullptr,
                                        1, N, D, 0.088f, 128, 64, nullptr) == TRA_ERR_INVALID_ARG,
              "sparse fp8, no kv_count");
        // schedules: a short grid takes the longest-first order, a long one the band order
        std::vector<int32_t> order(nqb);
        CHECK(tra_sparse_schedule(cnt.data(), 1, F, H, W, 128, 64, 8, 8, order.data(), nqb, nullptr) == TRA_OK &&
                  g_sched.lpt && g_sched.nqb == nqb && g_sched.nkb == nkb,
              "schedule (longest first)");
        {
            // the threshold: under 2 waves of 2 x 256 resident workgroups (1,024 rows) longest first,
            // from there the band order
            std::vector<int32_t> cnt_t((size_t)128 * nqb, 2), order_t((size_t)128 * nqb);
            CHECK(tra_sparse_schedule(cnt_t.data(), 127, F, H, W, 128, 64, 8, 8, order_t.data(),
                                      (int64_t)order_t.size(), nullptr) == TRA_OK && g_sched.lpt,
                  "schedule, 1,016 rows: longest first");
            CHECK(tra_sparse_schedule(cnt_t.data(), 128, F, H, W, 128, 64, 8, 8, order_t.data(),
                                      (int64_t)order_t.size(), nullptr) == TRA_OK && !g_sched.lpt,
                  "schedule, 1,024 rows: band order");
        }
        CHECK(tra_sparse_schedule(cnt.data(), 1, F, H, W, 128, 64, 8, 8, order.data(), nqb - 1, nullptr) ==
                  TRA_ERR_CAPACITY,
              "schedule capacity");
        CHECK(tra_block_sparse_attn_scheduled(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(),
                                              order.data(), 1, N, D, TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_OK &&
                  g_attn.order == order.data(),
              "scheduled sparse");
        CHECK(tra_block_sparse_attn_scheduled(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(),
                                              nullptr, 1, N, D, TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_ERR_INVALID_ARG,
              "scheduled sparse without an order");
        CHECK(tra_block_sparse_attn(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1, N, 96,
                                    TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_ERR_UNSUPPORTED,
              "D = 96");
        // a head's K and V are read as raw buffers: 2^31 bytes or more is refused before any launch
        // (nothing is read: the stand-in launchers never run for these)
        const int big = 1 << 23;  // 2^23 tokens x 128 x 2 B = 2^31 B
        CHECK(tra_block_sparse_attn(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1, big, D,
                                    TRA_BF16, 0.088f, 128, 64, nullptr) == TRA_ERR_UNSUPPORTED,
              "sparse, 2^31-byte head");
        CHECK(tra_block_sparse_attn_scheduled(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(),
                                              order.data(), 1, big, D, TRA_BF16, 0.088f, 128, 64,
                                              nullptr) == TRA_ERR_UNSUPPORTED,
              "scheduled sparse, 2^31-byte head");
        CHECK(tra_block_sparse_attn_fp8(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), nullptr,
                                        1, big, D, 0.088f, 128, 64, nullptr) == TRA_ERR_UNSUPPORTED,
              "fp8 sparse, 2^31-byte head");
        CHECK(tra_dense_attn_entropy(q.data(), k.data(), v.data(), o.data(), nullptr, nullptr, 1, big, D, TRA_BF16,
                                     0.088f, nullptr) == TRA_OK,
              "dense, 2^31-byte head (global loads: no buffer limit)");
        // the natural-order calls too (the sparse one forms its copy offsets within a head in 32-bit
        // signed arithmetic): 1 x 2048 x 4096 = 2^23 tokens is refused, 1 x 2047 x 4096 accepted
        CHECK(tra_natural_prepare(1, 2048, 4096, 8, 8) == TRA_ERR_UNSUPPORTED, "natural prepare, 2^31-byte head");
        CHECK(tra_block_sparse_attn_natural(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 1,
                                            1, 2048, 4096, D, TRA_BF16, 0.088f, 128, 64, 8, 8,
                                            nullptr) == TRA_ERR_UNSUPPORTED,
              "natural sparse, 2^31-byte head");
        CHECK(tra_dense_attn_entropy_natural(q.data(), k.data(), v.data(), o.data(), nullptr, nullptr, 1, 1, 2048, 4096,
                                             D, TRA_BF16, 0.088f, 8, 8, nullptr) == TRA_ERR_UNSUPPORTED,
              "natural dense, 2^31-byte head");
        CHECK(tra_natural_prepare(1, 2047, 4096, 8, 8) == TRA_OK, "natural prepare, largest head");
        CHECK(tra_dense_attn_entropy(nullptr, k.data(), v.data(), o.data(), nullptr, nullptr, 1, N, D, TRA_BF16,
                                     0.088f, nullptr) == TRA_ERR_INVALID_ARG,
              "null q");
    }
        // a long grid (21 x 45 x 80, 40 heads) takes the spatial band order: the table is a permutation of
    // one head's q-blocks, ordered by (row of tiles, frame, position along it)
    {
        const int F = 21, H = 45, W = 80, N = F * H * W, nqb = (N + 127) / 128, outer = 40;
        std::vector<int32_t> cnt((size_t)outer * nqb, 5), order((size_t)outer * nqb);
        CHECK(tra_sparse_schedule(cnt.data(), outer, F, H, W, 128, 64, 8, 8, order.data(), (int64_t)order.size(),
                                  nullptr) == TRA_OK && !g_sched.lpt && g_sched.band != nullptr,
              "schedule (band)");
        std::vector<int> seen(nqb, 0);
        int prev_band = -1, prev_frame = -1;
        for (int r = 0; r < nqb; ++r) {
            const int qb = g_sched.band[r];
            CHECK(qb >= 0 && qb < nqb && !seen[qb], "band table is a permutation");
            seen[qb] = 1;
            const int p0 = std::min(qb * 128 + 64, N - 1), f = p0 / (H * W), band = (p0 % (H * W)) / (8 * W);
            CHECK(band > prev_band || (band == prev_band && f >= prev_frame), "band table order");
            prev_band = band;
            prev_frame = f;
        }
    }
    // the 1D-distance mask: tables (ln t for t < N, k-block bounds) reach the launcher
    {
        const int F = 3, H = 15, W = 17, N = F * H * W, nqb = (N + 127) / 128, nkb = (N + 63) / 64;
        std::vector<float> ent((size_t)2 * N, 4.0f);
        std::vector<int32_t> cnt((size_t)2 * nqb), idx((size_t)2 * nqb * nkb);
        CHECK(tra_mask_prepare_1d(F, H, W, 0.05f, 128, 64, 8, 8) == TRA_OK, "mask_prepare_1d");
        CHECK(tra_build_block_mask_1d(ent.data(), 2, F, H, W, 0.05f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                      (int64_t)idx.size(), nullptr, nullptr) == TRA_OK,
              "build_block_mask_1d");
        CHECK(g_win_args.nqb == nqb && g_win_args.nkb == nkb && g_win_args.t.lnTmax == std::log((double)(N - 1)),
              "1d mask args");
        for (int kb = 0; kb < nkb; ++kb) {
            int lo = INT32_MAX, hi = -1;
            tra::TileGeom g{F, H, W, 8, 8, H * W, N};
            for (int p = kb * 64; p < std::min(N, kb * 64 + 64); ++p) {
                lo = std::min(lo, tra::tile_major_to_natural(p, g));
                hi = std::max(hi, tra::tile_major_to_natural(p, g));
            }
            CHECK(g_win_args.t.hull[kb].x == lo && g_win_args.t.hull[kb].y == hi, "k-block natural bounds");
        }
        CHECK(tra_build_block_mask_1d(ent.data(), 2, F, H, W, 0.0f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                      (int64_t)idx.size(), nullptr, nullptr) == TRA_ERR_INVALID_ARG,
              "1d mask, tau = 0");
        CHECK(tra_build_block_mask_1d(ent.data(), 2, F, H, W, 0.05f, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                      (int64_t)idx.size() - 1, nullptr, nullptr) == TRA_ERR_CAPACITY,
              "1d mask capacity");
        CHECK(tra_build_block_mask_1d(ent.data(), 2, F, H, W, 0.05f, 96, 64, 1, 8, 8, cnt.data(), idx.data(),
                                      (int64_t)idx.size(), nullptr, nullptr) == TRA_ERR_UNSUPPORTED,
              "1d mask, block_q = 96");
    }
    // after the prepare calls, every call of the step for that geometry allocates, copies and
    // queries nothing (so a caller may record the step into a HIP graph by stream capture)
    {
        const int F = 5, H = 24, W = 40, N = F * H * W, D = 128, nqb = (N + 127) / 128, nkb = (N + 63) / 64;
        const float tau = 0.04f, gamma = 0.5f, sc = 0.088f;
        CHECK(tra_mask_prepare(F, H, W, tau, gamma, 128, 64, 8, 8) == TRA_OK, "prepare (step)");
        CHECK(tra_mask_prepare_1d(F, H, W, tau, 128, 64, 8, 8) == TRA_OK, "prepare 1d (step)");
        CHECK(tra_natural_prepare(F, H, W, 8, 8) == TRA_OK, "natural prepare (step)");
        const int m0 = g_mallocs, c0 = g_copies, a0 = g_attrs, l0 = g_launches;
        std::vector<uint16_t> q((size_t)2 * N * D), k(q.size()), v(q.size()), t(q.size()), o(q.size());
        std::vector<float> ent((size_t)2 * N, 6.0f), lse((size_t)2 * N);
        std::vector<int32_t> cnt((size_t)2 * nqb, 3), idx((size_t)2 * nqb * nkb, 0), order((size_t)2 * nqb);
        const int outer_band = 256;  // 256 x 38 rows: past 2 waves of 2 x 256 workgroups, the band order
        std::vector<int32_t> cnt_band((size_t)outer_band * nqb, 3), order_band((size_t)outer_band * nqb);
        CHECK(tra_tile_major_permute(q.data(), t.data(), 2, F, H, W, D, TRA_BF16, 8, 8, nullptr) == TRA_OK, "step permute");
        CHECK(tra_dense_attn_entropy(t.data(), k.data(), v.data(), o.data(), ent.data(), lse.data(), 2, N, D, TRA_BF16,
                                     sc, nullptr) == TRA_OK, "step dense");
        CHECK(tra_build_block_mask(ent.data(), 2, F, H, W, tau, gamma, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                   (int64_t)idx.size(), nullptr, nullptr) == TRA_OK, "step mask");
        CHECK(tra_build_block_mask_1d(ent.data(), 2, F, H, W, tau, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                      (int64_t)idx.size(), nullptr, nullptr) == TRA_OK, "step 1d mask");
        CHECK(tra_sparse_schedule(cnt.data(), 2, F, H, W, 128, 64, 8, 8, order.data(), (int64_t)order.size(),
                                  nullptr) == TRA_OK && g_sched.lpt, "step schedule (longest first)");
        CHECK(tra_sparse_schedule(cnt_band.data(), outer_band, F, H, W, 128, 64, 8, 8, order_band.data(),
                                  (int64_t)order_band.size(), nullptr) == TRA_OK && !g_sched.lpt,
              "step schedule (band)");
        CHECK(tra_block_sparse_attn_scheduled(t.data(), k.data(), v.data(), o.data(), lse.data(), cnt.data(),
                                              idx.data(), order.data(), 2, N, D, TRA_BF16, sc, 128, 64,
                                              nullptr) == TRA_OK, "step scheduled sparse");
        CHECK(tra_tile_major_unpermute(o.data(), t.data(), 2, F, H, W, D, TRA_BF16, 8, 8, nullptr) == TRA_OK,
              "step unpermute");
        CHECK(tra_dense_attn_entropy_mask(t.data(), k.data(), v.data(), o.data(), ent.data(), nullptr, 2, F, H, W, D,
                                          TRA_BF16, sc, tau, gamma, 128, 64, 1, 8, 8, cnt.data(), idx.data(),
                                          (int64_t)idx.size(), nullptr, nullptr) == TRA_OK, "step fused");
        CHECK(tra_dense_attn_entropy_natural(q.data(), k.data(), v.data(), o.data(), ent.data(), nullptr, 2, F, H, W,
                                             D, TRA_BF16, sc, 8, 8, nullptr) == TRA_OK, "step natural dense");
        CHECK(tra_dense_attn_entropy_mask_natural(q.data(), k.data(), v.data(), o.data(), ent.data(), nullptr, 2, F, H,
                                                  W, D, TRA_BF16, sc, tau, gamma, 128, 64, 1, 8, 8, cnt.data(),
                                                  idx.data(), (int64_t)idx.size(), nullptr, nullptr) == TRA_OK,
              "step natural fused");
        CHECK(tra_block_sparse_attn_natural(q.data(), k.data(), v.data(), o.data(), nullptr, cnt.data(), idx.data(), 2,
                                            F, H, W, D, TRA_BF16, sc, 128, 64, 8, 8, nullptr) == TRA_OK &&
                  g_attn.band != nullptr, "step natural sparse");
        CHECK(g_launches - l0 == 12, "step launches");
        CHECK(g_mallocs == m0 && g_copies == c0 && g_attrs == a0, "no allocation, copy or query after prepare");
    }
    CHECK(g_launches == 27, "launch count");
    std::printf("host sanitize ok\n");
    return 0;
}
