// tra_api.cpp -- the C ABI of libtra.so: argument validation (before any HIP call),
// the per-device cache of mask tables, and dispatch to the HIP kernels.
//
// The host-built tables follow "Token Radius Attention for Efficient Video
// Generation", section 2 (Insight I budget tau * exp(H_i) / N, Insight II radius
// with per-frame factor exp(-gamma * delta)); the disk test is evaluated on the
// device as an integer comparison against these fp64 tables.
#include "../../include/tra.h"
#include "tra_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

namespace {

using tra::TileGeom;

constexpr int64_t kMaxN = (int64_t)1 << 30;

// Maps a HIP status to TRA_ERR_HIP; with TRA_DEBUG set in the environment the HIP
// error string goes to stderr.
tra_status from_hip(hipError_t e, const char *where) {
    if (e == hipSuccess) return TRA_OK;
    static const bool debug = std::getenv("TRA_DEBUG") != nullptr;
    if (debug) std::fprintf(stderr, "tra: %s: %s (%d)\n", where, hipGetErrorString(e), (int)e);
    return TRA_ERR_HIP;
}

// The kernels report launch failures through hipGetLastError(); an error left
// pending by earlier, unrelated runtime calls is cleared first so that it is not
// reported as ours.
void clear_pending_error() { (void)hipGetLastError(); }

bool valid_dtype(tra_dtype dt) { return dt == TRA_F32 || dt == TRA_BF16; }
int64_t dtype_bytes(tra_dtype dt) { return dt == TRA_F32 ? 4 : 2; }

tra_status check_grid(int F, int H, int W, int tile_h, int tile_w, TileGeom &g) {
    if (F < 1 || H < 1 || W < 1 || tile_h < 1 || tile_w < 1) return TRA_ERR_INVALID_ARG;
    const int64_t N = (int64_t)F * H * W;
    if (N > kMaxN || (int64_t)tile_h * W > kMaxN) return TRA_ERR_UNSUPPORTED;
    g.F = F; g.H = H; g.W = W; g.th = tile_h; g.tw = tile_w;
    g.HW = H * W;
    g.N = (int)N;
    return TRA_OK;
}

// ------------------------------------------------------------------ mask tables
// lambda[f][f'] = (ln tau - (2 gamma)|f - f'|) - ln(pi * S_f), S_f summed over f' in
// increasing order; lnT[t] = ln t.  Written with separately rounded fp64 operations
// (no contraction) so the tables are reproducible bit for bit with the C library.
#pragma clang fp contract(off)
void build_lambda(int F, double tau, double gamma, std::vector<double> &lam) {
    std::vector<double> S((size_t)F);
    for (int f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int fp = 0; fp < F; ++fp) {
            const int delta = f > fp ? f - fp : fp - f;
            acc += std::exp(-(2.0 * gamma) * (double)delta);
        }
        S[(size_t)f] = acc;
    }
    lam.resize((size_t)F * F);
    for (int f = 0; f < F; ++f)
        for (int fp = 0; fp < F; ++fp) {
            const int delta = f > fp ? f - fp : fp - f;
            lam[(size_t)f * F + fp] = (std::log(tau) - (2.0 * gamma) * (double)delta) - std::log(M_PI * S[(size_t)f]);
        }
}

void build_log_table(int tmax, std::vector<double> &lnT) {
    lnT.resize((size_t)tmax + 1);
    lnT[0] = -INFINITY;
    for (int t = 1; t <= tmax; ++t) lnT[(size_t)t] = std::log((double)t);
}
#pragma clang fp contract(on)

// k-block kb = tile-major positions [kb*bk, min(N, kb*bk + bk)) as a union of
// axis-aligned rectangles in (frame, row, column): maximal runs along a row are
// merged with the run directly above them when they span the same columns.
void build_rects(const TileGeom &g, int bk, std::vector<int32_t> &off, std::vector<int4> &rects) {
    const int nkb = (g.N + bk - 1) / bk;
    off.assign((size_t)nkb + 1, 0);
    rects.clear();
    for (int kb = 0; kb < nkb; ++kb) {
        off[(size_t)kb] = (int32_t)rects.size();
        const int p0 = kb * bk, p1 = std::min(g.N, p0 + bk);
        const size_t first = rects.size();
        int p = p0;
        while (p < p1) {
            int f, y, x;
            tra::tile_major_coords(p, g, f, y, x);
            int x1 = x;
            int q = p + 1;
            while (q < p1) {
                int f2, y2, xx2;
                tra::tile_major_coords(q, g, f2, y2, xx2);
                if (f2 != f || y2 != y || xx2 != x1 + 1) break;
                x1 = xx2;
                ++q;
            }
            // merge with an earlier rectangle of this block that ends on the row above
            bool merged = false;
            for (size_t r = first; r < rects.size(); ++r) {
                int4 &rc = rects[r];
                const int rx0 = rc.y >> 16, ry1 = rc.z & 0xffff, rx1 = rc.z >> 16;
                if (rc.x == f && ry1 == y - 1 && rx0 == x && rx1 == x1) {
                    rc.z = y | (x1 << 16);
                    merged = true;
                    break;
                }
            }
            if (!merged) rects.push_back(make_int4(f, y | (x << 16), y | (x1 << 16), 0));
            p = q;
        }
    }
    off[(size_t)nkb] = (int32_t)rects.size();
}

// The rectangles of every k-block at a fixed stride of rmax slots (rmax = most rectangles in one
// k-block), unused slots marked with frame -1; a used slot has w = f.
void build_rect_slots(const TileGeom &g, int bk, std::vector<int4> &slots, int &rmax) {
    std::vector<int32_t> off;
    std::vector<int4> rects;
    build_rects(g, bk, off, rects);
    const size_t nkb = off.size() - 1;
    rmax = 1;
    for (size_t kb = 0; kb < nkb; ++kb) rmax = std::max(rmax, off[kb + 1] - off[kb]);
    slots.assign(nkb * (size_t)rmax, make_int4(-1, 0, 0, -1));
    for (size_t kb = 0; kb < nkb; ++kb)
        for (int r = off[kb]; r < off[kb + 1]; ++r) {
            int4 rc = rects[(size_t)r];
            rc.w = rc.x;
            slots[kb * (size_t)rmax + (size_t)(r - off[kb])] = rc;
        }
}

struct TableKey {
    int dev, F, H, W, bk, th, tw;
    uint32_t tau_bits, gamma_bits;
    bool operator<(const TableKey &o) const {
        return std::tie(dev, F, H, W, bk, th, tw, tau_bits, gamma_bits) <
               std::tie(o.dev, o.F, o.H, o.W, o.bk, o.th, o.tw, o.tau_bits, o.gamma_bits);
    }
};

struct TableEntry {
    void *mem = nullptr;
    tra::MaskTables t{};
};

std::mutex g_mu;
std::map<TableKey, TableEntry> g_tables;

uint32_t fbits(float v) {
    uint32_t b;
    std::memcpy(&b, &v, 4);
    return b;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Inserts an uploaded table into its cache; on failure (std::bad_alloc from the map) frees the
// device copy, so no exception leaves the library and nothing leaks.
template <class Map, class Key, class Val>
tra_status cache_insert(Map &m, const Key &key, const Val &val, void *mem) {
    try {
        m.emplace(key, val);
    } catch (const std::bad_alloc &) {
        (void)hipFree(mem);
        return TRA_ERR_CAPACITY;
    }
    return TRA_OK;
}

tra_status get_tables(const TileGeom &g, float tau, float gamma, int bk, tra::MaskTables &out) {
    int dev = 0;
    const hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return from_hip(de, "hipGetDevice");
    const TableKey key{dev, g.F, g.H, g.W, bk, g.th, g.tw, fbits(tau), fbits(gamma)};
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_tables.find(key);
    if (it != g_tables.end()) {
        out = it->second.t;
        return TRA_OK;
    }
    std::vector<double> lam, lnT;
    std::vector<int4> slots;
    std::vector<char> host;
    int rmax = 1;
    const int tmax = (g.H - 1) * (g.H - 1) + (g.W - 1) * (g.W - 1);
    size_t b_lam = 0, b_lnT = 0, b_rect = 0;
    try {
        build_lambda(g.F, (double)tau, (double)gamma, lam);
        build_log_table(tmax, lnT);
        build_rect_slots(g, bk, slots, rmax);
        b_lam = align256(lam.size() * sizeof(double));
        b_lnT = align256(lnT.size() * sizeof(double));
        b_rect = align256(slots.size() * sizeof(int4));
        host.assign(b_lam + b_lnT + b_rect, 0);
    } catch (const std::bad_alloc &) {
        return TRA_ERR_CAPACITY;
    }
    std::memcpy(host.data(), lam.data(), lam.size() * sizeof(double));
    std::memcpy(host.data() + b_lam, lnT.data(), lnT.size() * sizeof(double));
    std::memcpy(host.data() + b_lam + b_lnT, slots.data(), slots.size() * sizeof(int4));
    void *mem = nullptr;
    const hipError_t me = hipMalloc(&mem, host.size());
    if (me != hipSuccess) return from_hip(me, "hipMalloc of mask tables");
    const hipError_t ce = hipMemcpy(mem, host.data(), host.size(), hipMemcpyHostToDevice);
    if (ce != hipSuccess) {
        (void)hipFree(mem);
        return from_hip(ce, "upload of mask tables");
    }
    TableEntry e;
    e.mem = mem;
    char *base = static_cast<char *>(mem);
    e.t.lam = reinterpret_cast<const double *>(base);
    e.t.lnT = reinterpret_cast<const double *>(base + b_lam);
    e.t.rects = reinterpret_cast<const int4 *>(base + b_lam + b_lnT);
    e.t.tmax = tmax;
    e.t.lnTmax = lnT[(size_t)tmax];
    e.t.rmax = rmax;
    const tra_status ins = cache_insert(g_tables, key, e, mem);
    if (ins != TRA_OK) return ins;
    out = e.t;
    return TRA_OK;
}

// ------------------------------------------------------------------ 1D-distance tables
// ln t for t < N, mu = ln tau - ln 2 (the window 2 d <= tau exp(H)), each k-block's natural-index
// hull and its rectangles; fp64 with the C library, no contraction.
#pragma clang fp contract(off)
double window_mu(double tau) { return std::log(tau) - std::log(2.0); }
#pragma clang fp contract(on)

std::map<TableKey, std::pair<void *, tra::WindowTables>> g_window;

tra_status get_window_tables(const TileGeom &g, float tau, int bk, tra::WindowTables &out) {
    int dev = 0;
    const hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return from_hip(de, "hipGetDevice");
    const TableKey key{dev, g.F, g.H, g.W, bk, g.th, g.tw, fbits(tau), 0u};
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_window.find(key);
    if (it != g_window.end()) {
        out = it->second.second;
        return TRA_OK;
    }
    std::vector<double> lnT;
    std::vector<int4> slots;
    std::vector<int2> hull;
    std::vector<char> host;
    int rmax = 1;
    const int nkb = (g.N + bk - 1) / bk;
    try {
        build_log_table(g.N - 1, lnT);
        build_rect_slots(g, bk, slots, rmax);
        hull.assign((size_t)nkb, make_int2(INT32_MAX, -1));
    } catch (const std::bad_alloc &) {
        return TRA_ERR_CAPACITY;
    }
    for (int kb = 0; kb < nkb; ++kb)
        for (int r = 0; r < rmax; ++r) {
            const int4 rc = slots[(size_t)kb * rmax + r];
            if (rc.w < 0) continue;
            const int y0 = rc.y & 0xffff, x0 = rc.y >> 16, y1 = rc.z & 0xffff, x1 = rc.z >> 16;
            int2 &h = hull[(size_t)kb];
            h.x = std::min(h.x, (rc.x * g.H + y0) * g.W + x0);
            h.y = std::max(h.y, (rc.x * g.H + y1) * g.W + x1);
        }
    const size_t b_lnT = align256(lnT.size() * sizeof(double));
    const size_t b_hull = align256(hull.size() * sizeof(int2));
    const size_t b_rect = align256(slots.size() * sizeof(int4));
    try {
        host.assign(b_lnT + b_hull + b_rect, 0);
    } catch (const std::bad_alloc &) {
        return TRA_ERR_CAPACITY;
    }
    std::memcpy(host.data(), lnT.data(), lnT.size() * sizeof(double));
    std::memcpy(host.data() + b_lnT, hull.data(), hull.size() * sizeof(int2));
    std::memcpy(host.data() + b_lnT + b_hull, slots.data(), slots.size() * sizeof(int4));
    void *mem = nullptr;
    const hipError_t me = hipMalloc(&mem, host.size());
    if (me != hipSuccess) return from_hip(me, "hipMalloc of window tables");
    const hipError_t ce = hipMemcpy(mem, host.data(), host.size(), hipMemcpyHostToDevice);
    if (ce != hipSuccess) {
        (void)hipFree(mem);
        return from_hip(ce, "upload of window tables");
    }
    tra::WindowTables t{};
    char *base = static_cast<char *>(mem);
    t.lnT = reinterpret_cast<const double *>(base);
    t.hull = reinterpret_cast<const int2 *>(base + b_lnT);
    t.rects = reinterpret_cast<const int4 *>(base + b_lnT + b_hull);
    t.lnTmax = lnT[(size_t)g.N - 1];
    t.mu = window_mu((double)tau);
    t.rmax = rmax;
    const tra_status ins = cache_insert(g_window, key, std::make_pair(mem, t), mem);
    if (ins != TRA_OK) return ins;
    out = t;
    return TRA_OK;
}

tra_status check_window_args(int F, int H, int W, float tau, int block_q, int block_k, int tile_h, int tile_w,
                             TileGeom &g) {
    const tra_status st = check_grid(F, H, W, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    if (!(tau > 0.0f) || !std::isfinite(tau)) return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if ((block_q != 64 && block_q != 128) || block_k != 64) return TRA_ERR_UNSUPPORTED;
    if (H > 32767 || W > 32767 || F > 32767) return TRA_ERR_UNSUPPORTED;  // rectangle bounds packed in 16 bits
    return TRA_OK;
}

// ------------------------------------------------------------------ natural-order map
// nat4[g] = natural row of tile-major position 4 g, for kernels that read and write
// natural-order tensors through the tile-major map.  Valid only when every aligned group
// of four tile-major positions is a run of four consecutive natural rows, which holds when
// W and the tile width are multiples of four; anything else is reported as unsupported
// (and checked here position by position).
struct NatKey {
    int dev, F, H, W, th, tw;
    bool operator<(const NatKey &o) const {
        return std::tie(dev, F, H, W, th, tw) < std::tie(o.dev, o.F, o.H, o.W, o.th, o.tw);
    }
};
std::map<NatKey, void *> g_nat;

tra_status get_nat_table(const TileGeom &g, const int32_t *&out) {
    if (g.W % 4 != 0 || g.tw % 4 != 0) return TRA_ERR_UNSUPPORTED;
    int dev = 0;
    const hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return from_hip(de, "hipGetDevice");
    const NatKey key{dev, g.F, g.H, g.W, g.th, g.tw};
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_nat.find(key);
    if (it != g_nat.end()) {
        out = static_cast<const int32_t *>(it->second);
        return TRA_OK;
    }
    std::vector<int32_t> nat4;
    try {
        nat4.resize((size_t)g.N / 4);
    } catch (const std::bad_alloc &) {
        return TRA_ERR_CAPACITY;
    }
    for (int q = 0; q < g.N / 4; ++q) {
        const int n0 = tra::tile_major_to_natural(4 * q, g);
        for (int j = 1; j < 4; ++j)
            if (tra::tile_major_to_natural(4 * q + j, g) != n0 + j) return TRA_ERR_UNSUPPORTED;
        nat4[(size_t)q] = n0;
    }
    void *mem = nullptr;
    const hipError_t me = hipMalloc(&mem, std::max<size_t>(1, nat4.size()) * sizeof(int32_t));
    if (me != hipSuccess) return from_hip(me, "hipMalloc of the natural-order map");
    const hipError_t ce = hipMemcpy(mem, nat4.data(), nat4.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (ce != hipSuccess) {
        (void)hipFree(mem);
        return from_hip(ce, "upload of the natural-order map");
    }
    const tra_status ins = cache_insert(g_nat, key, mem, mem);
    if (ins != TRA_OK) return ins;
    out = static_cast<const int32_t *>(mem);
    return TRA_OK;
}

// ------------------------------------------------------------------ schedule tables
// band[rank] = the q-block of one head at rank `rank` of the spatial band order: q-blocks sorted by
// (row of tiles, frame, position along the row of tiles) of their centre token, then by index.
struct BandKey {
    int dev, F, H, W, bq, th, tw;
    bool operator<(const BandKey &o) const {
        return std::tie(dev, F, H, W, bq, th, tw) < std::tie(o.dev, o.F, o.H, o.W, o.bq, o.th, o.tw);
    }
};
std::map<BandKey, void *> g_band;
std::map<int, int> g_cus;  // device -> compute units

tra_status get_band_table(const TileGeom &g, int bq, const int32_t *&out) {
    int dev = 0;
    const hipError_t de = hipGetDevice(&dev);
    if (de != hipSuccess) return from_hip(de, "hipGetDevice");
    const BandKey key{dev, g.F, g.H, g.W, bq, g.th, g.tw};
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_band.find(key);
    if (it != g_band.end()) {
        out = static_cast<const int32_t *>(it->second);
        return TRA_OK;
    }
    const int nqb = (g.N + bq - 1) / bq;
    std::vector<std::tuple<int, int, int, int>> keys;
    std::vector<int32_t> band;
    try {
        keys.reserve((size_t)nqb);
        band.resize((size_t)nqb);
    } catch (const std::bad_alloc &) {
        return TRA_ERR_CAPACITY;
    }
    const int span = g.th * g.W;  // tokens in one full row of tiles
    for (int qb = 0; qb < nqb; ++qb) {
        const int p0 = std::min(qb * bq + bq / 2, g.N - 1);
        const int f = p0 / g.HW, r = p0 - f * g.HW;
        keys.emplace_back(r / span, f, r % span, qb);
    }
    std::sort(keys.begin(), keys.end());
    for (int i = 0; i < nqb; ++i) band[(size_t)i] = std::get<3>(keys[(size_t)i]);
    void *mem = nullptr;
    const hipError_t me = hipMalloc(&mem, band.size() * sizeof(int32_t));
    if (me != hipSuccess) return from_hip(me, "hipMalloc of the band order");
    const hipError_t ce = hipMemcpy(mem, band.data(), band.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (ce != hipSuccess) {
        (void)hipFree(mem);
        return from_hip(ce, "upload of the band order");
    }
    const tra_status ins = cache_insert(g_band, key, mem, mem);
    if (ins != TRA_OK) return ins;
    out = static_cast<const int32_t *>(mem);
    return TRA_OK;
}

tra_status compute_units(int &cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cus.find(dev);
    if (it == g_cus.end()) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return from_hip(e, "hipDeviceGetAttribute");
        cus = std::max(1, n);
        try {
            g_cus.emplace(dev, cus);
        } catch (const std::bad_alloc &) {
            // not cached; the count is still right for this call
        }
        return TRA_OK;
    }
    cus = it->second;
    return TRA_OK;
}

// Grids of fewer than this many waves of resident sparse workgroups (two per compute unit) take the
// longest-first order: there the tail of unequal rows is a sizeable part of the call and there is
// little locality to keep.  From two waves up the band order's L2 locality is worth more (it ties
// longest first at 1.5 and 2.5 waves and beats it by 4-7% at 4 and 6 waves).
constexpr int kLptWaves = 2;
// Largest nkb the longest-first sort holds in its LDS histogram.
constexpr int kLptMaxBins = 16383;

// What tra_sparse_schedule looks up for this geometry and block_q: the band table and the
// device's compute-unit count, built ahead of a timed region or a stream capture.
tra_status prepare_schedule(const TileGeom &g, int block_q) {
    int cus = 0;
    const tra_status st = compute_units(cus);
    if (st != TRA_OK) return st;
    const int32_t *band = nullptr;
    return get_band_table(g, block_q, band);
}

// Checks shared by the natural-order attention entry points (after check_attn_common).
tra_status check_natural(int F, int H, int W, int D, tra_dtype dt, int tile_h, int tile_w, TileGeom &g) {
    const tra_status st = check_grid(F, H, W, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    if (dt != TRA_BF16 || D != 128) return TRA_ERR_UNSUPPORTED;
    if (W % 4 != 0 || tile_w % 4 != 0) return TRA_ERR_UNSUPPORTED;
    // the natural-order sparse kernel forms each copy's byte offset within a head in 32-bit
    // signed arithmetic (natural row * 256 + the offset within the run)
    if ((int64_t)g.N * D * 2 > (int64_t)INT32_MAX) return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

tra_status check_mask_args(int F, int H, int W, float tau, float gamma, int block_q, int block_k, int tile_h,
                           int tile_w, TileGeom &g) {
    const tra_status st = check_grid(F, H, W, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    if (!(tau > 0.0f) || !std::isfinite(tau) || !(gamma >= 0.0f) || !std::isfinite(gamma))
        return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if ((block_q != 64 && block_q != 128) || block_k != 64) return TRA_ERR_UNSUPPORTED;
    if (H > 32767 || W > 32767) return TRA_ERR_UNSUPPORTED;  // rectangle bounds are packed in 16 bits
    const int64_t tmax = (int64_t)(H - 1) * (H - 1) + (int64_t)(W - 1) * (W - 1);
    if (tmax > (int64_t)1 << 28) return TRA_ERR_UNSUPPORTED;
    if (F > 32767) return TRA_ERR_UNSUPPORTED;  // frame index packed in 16 bits of a list entry
    if (tra::mask_lds_bytes(block_q, F, g.HW) > 65536) return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

tra_status check_attn_common(const void *q, const void *k, const void *v, const void *o, int outer, int N, int D,
                             tra_dtype dt, float sm_scale) {
    if (!q || !k || !v || !o) return TRA_ERR_INVALID_ARG;
    if (outer < 1 || N < 1 || D < 1) return TRA_ERR_INVALID_ARG;
    if (!valid_dtype(dt)) return TRA_ERR_INVALID_ARG;
    if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return TRA_ERR_INVALID_ARG;
    if (o == q || o == k || o == v) return TRA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return TRA_ERR_UNSUPPORTED;
    if ((int64_t)N > kMaxN || (int64_t)outer * ((N + 63) / 64) > ((int64_t)1 << 31) - 1) return TRA_ERR_UNSUPPORTED;
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
    if (al % 16 != 0) return TRA_ERR_INVALID_ARG;  // rows are moved in 16-byte units
    return TRA_OK;
}



tra_status permute_impl(const void *src, void *dst, int outer, int F, int H, int W, int row_elems, tra_dtype dt,
                        int tile_h, int tile_w, hipStream_t s, int dir) {
    if (!src || !dst || src == dst) return TRA_ERR_INVALID_ARG;
    if (outer < 1 || row_elems < 1 || !valid_dtype(dt)) return TRA_ERR_INVALID_ARG;
    TileGeom g;
    const tra_status st = check_grid(F, H, W, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    if ((int64_t)outer * g.N > ((int64_t)1 << 40)) return TRA_ERR_UNSUPPORTED;
    clear_pending_error();
    return from_hip(tra::launch_permute(src, dst, outer, g, (int64_t)row_elems * dtype_bytes(dt), dir, s),
                    "permute");
}

// Mask arguments after check_mask_args succeeded: sizes, capacity, tables (first use uploads).
tra_status fill_mask_args(const TileGeom &g, const float *entropy, int outer, float tau, float gamma, int block_q,
                          int block_k, int vote_threshold, int32_t *kv_count, int32_t *kv_index,
                          int64_t kv_index_capacity, uint8_t *block_mask, tra::MaskArgs &m) {
    const int nqb = (g.N + block_q - 1) / block_q;
    const int nkb = (g.N + block_k - 1) / block_k;
    if ((int64_t)outer * nqb > ((int64_t)1 << 31) - 1) return TRA_ERR_UNSUPPORTED;
    if (kv_index_capacity < (int64_t)outer * nqb * nkb) return TRA_ERR_CAPACITY;
    m = tra::MaskArgs{};
    const tra_status st = get_tables(g, tau, gamma, block_k, m.t);
    if (st != TRA_OK) return st;
    m.ent = entropy;
    m.outer = outer; m.nqb = nqb; m.nkb = nkb;
    m.block_q = block_q; m.block_k = block_k; m.vote = vote_threshold;
    m.nqf_max = tra::mask_frames_per_qblock(block_q, g.HW, g.F);
    m.chunk = std::min(256, tra::kMaskEntryCap / std::max(1, m.t.rmax));
    m.g = g;
    m.kv_count = kv_count; m.kv_index = kv_index; m.block_mask = block_mask;
    return TRA_OK;
}

// Attention arguments (nqb / nkb for 128-query and 64-key blocks; a launcher may regroup).
tra::AttnArgs attn_args(const void *q, const void *k, const void *v, void *o, float *entropy, float *lse, int outer,
                        int N, float sm_scale) {
    tra::AttnArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.ent = entropy; a.lse = lse;
    a.outer = outer; a.N = N;
    a.nqb = (N + 127) / 128;
    a.nkb = (N + 63) / 64;
    a.sm_scale = sm_scale;
    a.c = (float)((double)sm_scale * 1.4426950408889634074);
    return a;
}

// The tile-major bf16 (and fp8-score) sparse kernels read each head's K and V as raw buffers,
// whose sizes are 32-bit signed byte counts.
tra_status check_head_buffers(int N, int D, tra_dtype dt) {
    if (dt == TRA_BF16 && (int64_t)N * D * 2 > (int64_t)INT32_MAX) return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

// The fused warm-up (dense attention + entropy + mask rows), tile-major or natural-order
// q, k, v, o.
tra_status dense_mask_impl(const void *q, const void *k, const void *v, void *o, float *entropy, float *lse, int outer,
                           int F, int H, int W, int D, tra_dtype dt, float sm_scale, float tau, float gamma,
                           int block_q, int block_k, int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                           int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask, hipStream_t s,
                           bool natural) {
    if (!kv_count || !kv_index || outer < 1 || vote_threshold < 1) return TRA_ERR_INVALID_ARG;
    TileGeom g;
    tra_status st = check_mask_args(F, H, W, tau, gamma, block_q, block_k, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    st = check_attn_common(q, k, v, o, outer, g.N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    if (dt != TRA_BF16 || D != 128 || block_q != 128 || block_k != 64) return TRA_ERR_UNSUPPORTED;
    if (!tra::mask_fits_split(block_q, F, g.HW)) return TRA_ERR_UNSUPPORTED;
    if (natural) {
        TileGeom gn;
        st = check_natural(F, H, W, D, dt, tile_h, tile_w, gn);
        if (st != TRA_OK) return st;
    }
    tra::MaskArgs m;
    st = fill_mask_args(g, entropy, outer, tau, gamma, block_q, block_k, vote_threshold, kv_count, kv_index,
                        kv_index_capacity, block_mask, m);
    if (st != TRA_OK) return st;
    tra::AttnArgs a = attn_args(q, k, v, o, entropy, lse, outer, g.N, sm_scale);
    if (natural) {
        st = get_nat_table(g, a.nat4);
        if (st != TRA_OK) return st;
    }
    clear_pending_error();
    return from_hip(tra::launch_dense_mask(a, m, s), natural ? "dense attention with mask (natural order)"
                                                            : "dense attention with mask");
}

}  // namespace

extern "C" {

const char *tra_status_string(tra_status st) {
    switch (st) {
        case TRA_OK: return "TRA_OK";
        case TRA_ERR_INVALID_ARG: return "TRA_ERR_INVALID_ARG";
        case TRA_ERR_UNSUPPORTED: return "TRA_ERR_UNSUPPORTED";
        case TRA_ERR_HIP: return "TRA_ERR_HIP";
        case TRA_ERR_CAPACITY: return "TRA_ERR_CAPACITY";
    }
    return "TRA_ERR_UNKNOWN";
}

tra_status tra_tile_major_permute(const void *x, void *y, int outer, int F, int H, int W, int row_elems,
                                  tra_dtype dt, int tile_h, int tile_w, hipStream_t s) {
    return permute_impl(x, y, outer, F, H, W, row_elems, dt, tile_h, tile_w, s, 0);
}

tra_status tra_tile_major_unpermute(const void *y, void *x, int outer, int F, int H, int W, int row_elems,
                                    tra_dtype dt, int tile_h, int tile_w, hipStream_t s) {
    return permute_impl(y, x, outer, F, H, W, row_elems, dt, tile_h, tile_w, s, 1);
}

tra_status tra_dense_attn_entropy(const void *q, const void *k, const void *v, void *o, float *entropy, float *lse,
                                  int outer, int N, int D, tra_dtype dt, float sm_scale, hipStream_t s) {
    const tra_status st = check_attn_common(q, k, v, o, outer, N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    const tra::AttnArgs a = attn_args(q, k, v, o, entropy, lse, outer, N, sm_scale);
    clear_pending_error();
    return from_hip(tra::launch_attention(a, D, dt == TRA_BF16 ? 1 : 0, 128, false, s), "dense attention");
}

tra_status tra_mask_prepare(int F, int H, int W, float tau, float gamma, int block_q, int block_k, int tile_h,
                            int tile_w) {
    TileGeom g;
    tra_status st = check_mask_args(F, H, W, tau, gamma, block_q, block_k, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    tra::MaskTables t;
    st = get_tables(g, tau, gamma, block_k, t);
    if (st != TRA_OK) return st;
    return prepare_schedule(g, block_q);
}

tra_status tra_mask_prepare_1d(int F, int H, int W, float tau, int block_q, int block_k, int tile_h, int tile_w) {
    TileGeom g;
    tra_status st = check_window_args(F, H, W, tau, block_q, block_k, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    tra::WindowTables t;
    st = get_window_tables(g, tau, block_k, t);
    if (st != TRA_OK) return st;
    return prepare_schedule(g, block_q);
}

tra_status tra_build_block_mask_1d(const float *entropy, int outer, int F, int H, int W, float tau, int block_q,
                                   int block_k, int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                   int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                   hipStream_t s) {
    if (!entropy || !kv_count || !kv_index || outer < 1 || vote_threshold < 1) return TRA_ERR_INVALID_ARG;
    TileGeom g;
    tra_status st = check_window_args(F, H, W, tau, block_q, block_k, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    const int nqb = (g.N + block_q - 1) / block_q, nkb = (g.N + block_k - 1) / block_k;
    if ((int64_t)outer * nqb > ((int64_t)1 << 31) - 1) return TRA_ERR_UNSUPPORTED;
    if (kv_index_capacity < (int64_t)outer * nqb * nkb) return TRA_ERR_CAPACITY;
    tra::WindowArgs a{};
    st = get_window_tables(g, tau, block_k, a.t);
    if (st != TRA_OK) return st;
    a.ent = entropy;
    a.outer = outer; a.nqb = nqb; a.nkb = nkb;
    a.block_q = block_q; a.block_k = block_k; a.vote = vote_threshold;
    a.g = g;
    a.kv_count = kv_count; a.kv_index = kv_index; a.block_mask = block_mask;
    clear_pending_error();
    return from_hip(tra::launch_build_mask_1d(a, s), "build 1D-distance mask");
}

tra_status tra_build_block_mask(const float *entropy, int outer, int F, int H, int W, float tau, float gamma,
                                int block_q, int block_k, int vote_threshold, int tile_h, int tile_w,
                                int32_t *kv_count, int32_t *kv_index, int64_t kv_index_capacity,
                                uint8_t *block_mask, hipStream_t s) {
    if (!entropy || !kv_count || !kv_index || outer < 1 || vote_threshold < 1) return TRA_ERR_INVALID_ARG;
    TileGeom g;
    tra_status st = check_mask_args(F, H, W, tau, gamma, block_q, block_k, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    tra::MaskArgs m;
    st = fill_mask_args(g, entropy, outer, tau, gamma, block_q, block_k, vote_threshold, kv_count, kv_index,
                        kv_index_capacity, block_mask, m);
    if (st != TRA_OK) return st;
    clear_pending_error();
    return from_hip(tra::launch_build_mask(m, s), "build mask");
}

tra_status tra_dense_attn_entropy_mask(const void *q, const void *k, const void *v, void *o, float *entropy,
                                       float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                       float sm_scale, float tau, float gamma, int block_q, int block_k,
                                       int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                       int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                       hipStream_t s) {
    return dense_mask_impl(q, k, v, o, entropy, lse, outer, F, H, W, D, dt, sm_scale, tau, gamma, block_q, block_k,
                           vote_threshold, tile_h, tile_w, kv_count, kv_index, kv_index_capacity, block_mask, s,
                           false);
}

tra_status tra_dense_attn_entropy_mask_natural(const void *q, const void *k, const void *v, void *o, float *entropy,
                                               float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                               float sm_scale, float tau, float gamma, int block_q, int block_k,
                                               int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                               int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                               hipStream_t s) {
    return dense_mask_impl(q, k, v, o, entropy, lse, outer, F, H, W, D, dt, sm_scale, tau, gamma, block_q, block_k,
                           vote_threshold, tile_h, tile_w, kv_count, kv_index, kv_index_capacity, block_mask, s,
                           true);
}

tra_status tra_natural_prepare(int F, int H, int W, int tile_h, int tile_w) {
    TileGeom g;
    tra_status st = check_natural(F, H, W, 128, TRA_BF16, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    const int32_t *map = nullptr;
    st = get_nat_table(g, map);
    if (st != TRA_OK) return st;
    const int32_t *band = nullptr;  // the natural sparse call's row order (block_q = 128)
    return get_band_table(g, 128, band);
}

tra_status tra_dense_attn_entropy_natural(const void *q, const void *k, const void *v, void *o, float *entropy,
                                          float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                          float sm_scale, int tile_h, int tile_w, hipStream_t s) {
    if (F < 1 || H < 1 || W < 1) return TRA_ERR_INVALID_ARG;
    const int64_t N = (int64_t)F * H * W;
    if (N > kMaxN) return TRA_ERR_UNSUPPORTED;
    tra_status st = check_attn_common(q, k, v, o, outer, (int)N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    TileGeom g;
    st = check_natural(F, H, W, D, dt, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    tra::AttnArgs a = attn_args(q, k, v, o, entropy, lse, outer, g.N, sm_scale);
    st = get_nat_table(g, a.nat4);
    if (st != TRA_OK) return st;
    clear_pending_error();
    return from_hip(tra::launch_attention_natural(a, false, s), "dense attention (natural order)");
}

tra_status tra_block_sparse_attn_natural(const void *q, const void *k, const void *v, void *o, float *lse,
                                         const int32_t *kv_count, const int32_t *kv_index, int outer, int F, int H,
                                         int W, int D, tra_dtype dt, float sm_scale, int block_q, int block_k,
                                         int tile_h, int tile_w, hipStream_t s) {
    if (F < 1 || H < 1 || W < 1) return TRA_ERR_INVALID_ARG;
    const int64_t N = (int64_t)F * H * W;
    if (N > kMaxN) return TRA_ERR_UNSUPPORTED;
    tra_status st = check_attn_common(q, k, v, o, outer, (int)N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    if (!kv_count || !kv_index) return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if (block_q != 128 || block_k != 64) return TRA_ERR_UNSUPPORTED;
    TileGeom g;
    st = check_natural(F, H, W, D, dt, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    tra::AttnArgs a = attn_args(q, k, v, o, nullptr, lse, outer, g.N, sm_scale);
    a.kv_count = kv_count; a.kv_index = kv_index;
    st = get_nat_table(g, a.nat4);
    if (st != TRA_OK) return st;
    // the geometry is known here: the workgroups take the rows in the spatial band order
    st = get_band_table(g, block_q, a.band);
    if (st != TRA_OK) return st;
    clear_pending_error();
    return from_hip(tra::launch_attention_natural(a, true, s), "sparse attention (natural order)");
}

tra_status tra_sparse_schedule(const int32_t *kv_count, int outer, int F, int H, int W, int block_q, int block_k,
                               int tile_h, int tile_w, int32_t *order, int64_t order_capacity, hipStream_t s) {
    if (!kv_count || !order || outer < 1) return TRA_ERR_INVALID_ARG;
    TileGeom g;
    tra_status st = check_grid(F, H, W, tile_h, tile_w, g);
    if (st != TRA_OK) return st;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if ((block_q != 64 && block_q != 128) || block_k != 64) return TRA_ERR_UNSUPPORTED;
    const int nqb = (g.N + block_q - 1) / block_q, nkb = (g.N + block_k - 1) / block_k;
    if ((int64_t)outer * nqb > ((int64_t)1 << 31) - 1) return TRA_ERR_UNSUPPORTED;
    if (order_capacity < (int64_t)outer * nqb) return TRA_ERR_CAPACITY;
    int cus = 0;
    st = compute_units(cus);
    if (st != TRA_OK) return st;
    tra::ScheduleArgs a{};
    a.kv_count = kv_count; a.order = order;
    a.outer = outer; a.nqb = nqb; a.nkb = nkb;
    a.lpt = (int64_t)outer * nqb < (int64_t)kLptWaves * 2 * cus && nkb <= kLptMaxBins;
    if (!a.lpt) {
        st = get_band_table(g, block_q, a.band);
        if (st != TRA_OK) return st;
    }
    clear_pending_error();
    return from_hip(tra::launch_schedule(a, s), "sparse schedule");
}

tra_status tra_block_sparse_attn_scheduled(const void *q, const void *k, const void *v, void *o, float *lse,
                                           const int32_t *kv_count, const int32_t *kv_index, const int32_t *order,
                                           int outer, int N, int D, tra_dtype dt, float sm_scale, int block_q,
                                           int block_k, hipStream_t s) {
    tra_status st = check_attn_common(q, k, v, o, outer, N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    st = check_head_buffers(N, D, dt);
    if (st != TRA_OK) return st;
    if (!kv_count || !kv_index || !order) return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if ((block_q != 64 && block_q != 128) || block_k != 64) return TRA_ERR_UNSUPPORTED;
    tra::AttnArgs a = attn_args(q, k, v, o, nullptr, lse, outer, N, sm_scale);
    a.kv_count = kv_count; a.kv_index = kv_index; a.order = order;
    a.nqb = (N + block_q - 1) / block_q;
    clear_pending_error();
    return from_hip(tra::launch_attention(a, D, dt == TRA_BF16 ? 1 : 0, block_q, true, s), "sparse attention (scheduled)");
}

tra_status tra_block_sparse_attn_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                                     const int32_t *kv_count, const int32_t *kv_index, const int32_t *order,
                                     int outer, int N, int D, float sm_scale, int block_q, int block_k,
                                     hipStream_t s) {
    // q and k are one byte per element, v and o bf16: the common checks hold for every one
    tra_status st = check_attn_common(q, k, v, o, outer, N, D, TRA_BF16, sm_scale);
    if (st != TRA_OK) return st;
    st = check_head_buffers(N, D, TRA_BF16);  // v is bf16
    if (st != TRA_OK) return st;
    if (!kv_count || !kv_index) return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if (D != 128 || block_q != 128 || block_k != 64) return TRA_ERR_UNSUPPORTED;
    tra::AttnArgs a = attn_args(q, k, v, o, nullptr, lse, outer, N, sm_scale);
    a.kv_count = kv_count; a.kv_index = kv_index; a.order = order;
    clear_pending_error();
    return from_hip(tra::launch_attention_fp8(a, s), "sparse attention (fp8 q, k)");
}

tra_status tra_block_sparse_attn(const void *q, const void *k, const void *v, void *o, float *lse,
                                 const int32_t *kv_count, const int32_t *kv_index, int outer, int N, int D,
                                 tra_dtype dt, float sm_scale, int block_q, int block_k, hipStream_t s) {
    tra_status st = check_attn_common(q, k, v, o, outer, N, D, dt, sm_scale);
    if (st != TRA_OK) return st;
    st = check_head_buffers(N, D, dt);
    if (st != TRA_OK) return st;
    if (!kv_count || !kv_index) return TRA_ERR_INVALID_ARG;
    if (block_q < 1 || block_k < 1) return TRA_ERR_INVALID_ARG;
    if ((block_q != 64 && block_q != 128) || block_k != 64) return TRA_ERR_UNSUPPORTED;
    tra::AttnArgs a = attn_args(q, k, v, o, nullptr, lse, outer, N, sm_scale);
    a.kv_count = kv_count; a.kv_index = kv_index;
    a.nqb = (N + block_q - 1) / block_q;
    clear_pending_error();
    return from_hip(tra::launch_attention(a, D, dt == TRA_BF16 ? 1 : 0, block_q, true, s), "sparse attention");
}

}  // extern "C"
