// tra_internal.h -- declarations shared by the C ABI layer and the HIP kernels of
// libtra.so.  Not part of the public interface (include/tra.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tra {

// Geometry of the latent grid and its tile-major order.
struct TileGeom {
    int F, H, W;      // frames, rows, columns
    int th, tw;       // tile shape
    int HW;           // H * W
    int N;            // F * H * W
};

// Position p of the tile-major sequence -> (frame, row, column) of that token.
// Tile-major order: frame, row of tiles, tile, row inside the tile, column inside
// the tile; edge tiles clipped.
__host__ __device__ inline void tile_major_coords(int p, const TileGeom &g, int &f, int &y, int &x) {
    f = p / g.HW;
    const int r = p - f * g.HW;
    const int band = g.th * g.W;                 // tokens in one full row of tiles
    const int ty = r / band;
    const int r2 = r - ty * band;
    const int ht = min(g.th, g.H - ty * g.th);   // rows in this row of tiles
    const int tile = ht * g.tw;                  // tokens in a full-width tile of this row
    const int tx = r2 / tile;
    const int r3 = r2 - tx * tile;
    const int wt = min(g.tw, g.W - tx * g.tw);   // columns in this tile
    const int yy = r3 / wt;
    y = ty * g.th + yy;
    x = tx * g.tw + (r3 - yy * wt);
}

__host__ __device__ inline int tile_major_to_natural(int p, const TileGeom &g) {
    int f, y, x;
    tile_major_coords(p, g, f, y, x);
    return (f * g.H + y) * g.W + x;
}

// ---------------------------------------------------------------- permute
// dir = 0: y[o][p] = x[o][pi(p)]; dir = 1: x[o][pi(p)] = y[o][p].
hipError_t launch_permute(const void *src, void *dst, int outer, const TileGeom &g, int64_t row_bytes,
                          int dir, hipStream_t s);

// ---------------------------------------------------------------- mask
// Device-resident tables for one (geometry, tau, gamma, block_k, tile) key.
struct MaskTables {
    const double *lam;      // [F][F]  (ln tau - (2 gamma)|f - f'|) - ln(pi S_f)
    const double *lnT;      // [tmax + 1], lnT[t] = ln t, lnT[0] = -inf
    const int4 *rects;      // [nkb][rmax] {f, y0 | x0 << 16, y1 | x1 << 16, f}: inclusive corners packed
                            // (row | col << 16); unused slots have x = w = -1
    double lnTmax;          // lnT[tmax]
    int tmax;               // (H-1)^2 + (W-1)^2
    int rmax;               // most rectangles in one k-block
};

// Rectangles the mask kernel can hold in LDS for its exact test per chunk of k-blocks.
constexpr int kMaskEntryCap = 768;
// Threads of one mask row's builder (a workgroup, or half of the fused kernel's).
constexpr int kMaskThreads = 256;

struct MaskArgs {
    const float *ent;
    int outer, nqb, nkb, block_q, block_k, vote;
    int nqf_max;      // most frames one q-block touches
    int chunk;        // k-blocks per chunk: min(256, kMaskEntryCap / rmax)
    TileGeom g;
    MaskTables t;
    int32_t *kv_count;
    int32_t *kv_index;
    uint8_t *block_mask;
};

hipError_t launch_build_mask(const MaskArgs &a, hipStream_t s);
int mask_frames_per_qblock(int block_q, int HW, int F);
size_t mask_lds_bytes(int block_q, int F, int HW);
// whether the mask state fits the four 16 KB tile buffers of the attention kernel (fused path)
bool mask_fits_split(int block_q, int F, int HW);

// 1D-distance variant: device tables for one (geometry, tau, block_k, tile) key.
struct WindowTables {
    const double *lnT;   // [N] ln t, lnT[0] = -inf
    const int2 *hull;    // [nkb] smallest and largest natural index of each k-block's tokens
    const int4 *rects;   // [nkb][rmax] k-block rectangles, as MaskTables::rects
    double lnTmax;       // lnT[N - 1]
    double mu;           // ln tau - ln 2
    int rmax;
};

struct WindowArgs {
    const float *ent;
    int outer, nqb, nkb, block_q, block_k, vote;
    TileGeom g;
    WindowTables t;
    int32_t *kv_count;
    int32_t *kv_index;
    uint8_t *block_mask;
};

hipError_t launch_build_mask_1d(const WindowArgs &a, hipStream_t s);

// ---------------------------------------------------------------- attention
// Block-sparse attention: the k-block a list entry e names, clamped into [0, nkb), so that any
// list value keeps every access inside k and v.  The ragged last k-block (N % 64 != 0) is then
// copied row by row and its rows past N are masked.
__host__ __device__ inline int sparse_kblock(int e, int nkb) { return min(max(e, 0), nkb - 1); }

// The k-block a copy issued between the S^T products fetches for list entry e.  Those copies
// move whole 64-row tiles and skip the ragged-tile masking, so the entry is clamped to the last
// full k-block (nfull = N / 64).  A valid list (ascending, distinct) holds the ragged k-block
// only as its last entry, which such copies never fetch, so valid lists are unaffected.
__host__ __device__ inline int sparse_full_kblock(int e, int nfull) { return min(max(e, 0), max(nfull - 1, 0)); }

// Number of leading steps of a sparse list walk of ntiles tiles whose copies run between the
// products: pairs of steps (j, j + 1) while j + 4 < ntiles.  Step j copies K of tile j + 2 and
// V of tile j + 1 and reads the list entry of tile j + 3; all are before the last tile.
__host__ __device__ inline int sparse_fast_steps(int ntiles) { return ntiles > 4 ? 2 * ((ntiles - 3) / 2) : 0; }

struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    float *ent, *lse;
    const int32_t *kv_count, *kv_index;
    // null: workgroups take the rows in the library's default order; otherwise workgroup b runs row
    // order[b] (clamped into [0, outer * nqb)), the order tra_sparse_schedule writes
    const int32_t *order;
    // without an order: null, or one head's q-blocks in the spatial band order (nqb entries), dealt to
    // the XCDs in runs as tra_sparse_schedule's band order
    const int32_t *band;
    int outer, N, nqb, nkb;
    float c;          // sm_scale * log2(e)
    float sm_scale;
    // null: q, k, v, o in tile-major order.  Otherwise they are in natural order and
    // nat4[g] is the natural row of tile-major position 4 g (every aligned group of four
    // tile-major positions is a run of four natural rows); entropy and lse stay tile-major.
    const int32_t *nat4;
};

// dtype: 0 = fp32, 1 = bf16.  sparse: walk kv_index; else every k-block (dense).
hipError_t launch_attention(const AttnArgs &a, int D, int dtype, int block_q, bool sparse, hipStream_t s);

// ---------------------------------------------------------------- schedule
// Rows per run of the spatial band order on one XCD (about the workgroups an XCD holds at once).
constexpr int kBandRun = 64;

// workgroup b -> position in the run order: XCD x = b mod 8 takes runs of kBandRun consecutive
// positions, the runs of the 8 XCDs advancing together; the ragged last row of runs keeps the
// identity (every position once)
__device__ inline int xcd_runs(int b, int total) {
    const int full = (total / (8 * kBandRun)) * (8 * kBandRun);
    if (b >= full) return b;
    const int x = b & 7, k = b >> 3;
    return (k / kBandRun) * (8 * kBandRun) + x * kBandRun + (k % kBandRun);
}

struct ScheduleArgs {
    const int32_t *kv_count;  // [outer][nqb] (longest-first order)
    const int32_t *band;      // [nqb]: one head's q-blocks in band order (band order)
    int32_t *order;           // [outer * nqb] out
    int outer, nqb, nkb;
    bool lpt;                 // longest first; else the spatial band order
};
hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s);

// block-sparse attention with fp8 (OCP e4m3) q and k, bf16 v and o: D = 128, 128-query blocks
hipError_t launch_attention_fp8(const AttnArgs &a, hipStream_t s);

// natural-order q, k, v, o (a.nat4 set): bf16, D = 128; sparse with 128-query blocks
hipError_t launch_attention_natural(const AttnArgs &a, bool sparse, hipStream_t s);

// dense attention + entropy with the mask builder as epilogue (bf16, D = 128, block_q = 128)
hipError_t launch_dense_mask(const AttnArgs &a, const MaskArgs &m, hipStream_t s);

}  // namespace tra
