/*
 * tra.h -- C ABI of libtra.so, the MI355X (gfx950) hot path of Token Radius
 * Attention (TRA).
 *
 * The method ("Token Radius Attention for Efficient Video Generation",
 * gist.science summary of arXiv 2608.02504, section 2): a dense warm-up
 * attention pass yields each query's softmax entropy H_i; the entropy maps to
 * a token budget tau * exp(H_i) (Insight I), the budget to a query-centred
 * spatial radius that shrinks with temporal distance by exp(-gamma * delta)
 * (Insight II); tokens are laid out tile-major, a fused kernel turns the
 * token-level disks into a regular block-sparse mask (distance computation,
 * radius comparison, block pruning, token voting), and later denoising steps
 * run block-sparse attention over that mask (TRA pipeline, steps 1-3).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps caller memory.
 *  - Tensors are [outer][N][row] contiguous (outer = batch * heads), row-major.
 *    Attention inputs and outputs, entropies and masks are in TILE-MAJOR token
 *    order (see tra_tile_major_permute).
 *  - Every call is asynchronous on the caller's stream `s` (0 = the null
 *    stream) and returns once the work is enqueued.  Nothing on these paths
 *    copies device data to the host.
 *  - Arguments are validated before any HIP call: a bad argument returns
 *    TRA_ERR_INVALID_ARG / TRA_ERR_UNSUPPORTED / TRA_ERR_CAPACITY and enqueues
 *    nothing.  A failing HIP call returns TRA_ERR_HIP.  No C++ exception
 *    crosses the ABI.
 *  - Library state: a per-device cache of small fp64 tables and block
 *    geometry for the mask builders, of the band order for the schedule, and
 *    of the tile-major map for the natural-order attention calls, guarded by a
 *    mutex.  Its first use for a geometry allocates and uploads them
 *    synchronously.  tra_mask_prepare, tra_mask_prepare_1d and
 *    tra_natural_prepare do that ahead of time: afterwards the calls for that
 *    geometry neither allocate nor copy between host and device, so they can
 *    run inside a timed region or be recorded into a HIP graph by stream
 *    capture.  Entries live until the process ends.
 */
#ifndef TRA_H_
#define TRA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRA_OK = 0,
    TRA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, N != F*H*W, tau <= 0, ... */
    TRA_ERR_UNSUPPORTED = 2, /* valid but not implemented: head dim, dtype or block shape */
    TRA_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    TRA_ERR_CAPACITY = 4     /* an output buffer is smaller than the call needs */
} tra_status;

typedef enum { TRA_F32 = 0, TRA_BF16 = 1 } tra_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char *tra_status_string(tra_status st);

/*
 * Tile-major permutation (TRA pipeline step 3, tile-major layout: tokens are
 * reordered so that spatial neighbours are contiguous in the sequence).
 *
 * Token order: natural index (f*H + h)*W + w.  Tile-major order walks frame
 * f, then rows of tiles, then tiles left to right, then rows inside the tile,
 * then columns inside the tile; tiles are tile_h x tile_w, clipped at the
 * bottom/right edges, never padded, so the map is a bijection on N = F*H*W.
 *
 *   permute:   y[o][p][:] = x[o][pi(p)][:]
 *   unpermute: x[o][pi(p)][:] = y[o][p][:]
 * where pi(p) is the natural index of the token at tile-major position p.
 *
 * x, y: device, [outer][N][row_elems] of `dt` (fp32 or bf16), distinct
 * buffers (in-place is rejected).  row_elems = 1 reorders a per-token vector
 * such as the entropies.  Pure data movement: bit-exact.
 */
tra_status tra_tile_major_permute(const void *x, void *y, int outer, int F, int H, int W, int row_elems,
                                  tra_dtype dt, int tile_h, int tile_w, hipStream_t s);
tra_status tra_tile_major_unpermute(const void *y, void *x, int outer, int F, int H, int W, int row_elems,
                                    tra_dtype dt, int tile_h, int tile_w, hipStream_t s);

/*
 * Dense warm-up attention with fused per-query entropy (section 1: dense 3D
 * self-attention over N video tokens; pipeline step 1: the entropy of every
 * query is taken during the dense warm-up; section 3 contribution 3: the
 * entropy kernel is fused to keep its overhead low).
 *
 *   o_i   = sum_j softmax_j(sm_scale * <q_i, k_j>) v_j      (all N keys, non-causal)
 *   H_i   = -sum_j p_ij ln p_ij                               (nats)
 *   lse_i = ln sum_j exp(sm_scale * <q_i, k_j>)
 *
 * q, k, v, o: device, [outer][N][D] of `dt` (the same dtype for all four);
 * D in {64, 128}.  bf16 inputs are multiplied on bf16 matrix cores with fp32
 * accumulation; softmax statistics and the entropy are fp32; fp32 inputs use
 * fp32 matrix cores.  entropy, lse: device fp32 [outer][N], each may be NULL.
 * o must not alias q, k or v.
 */
tra_status tra_dense_attn_entropy(const void *q, const void *k, const void *v, void *o, float *entropy,
                                  float *lse, int outer, int N, int D, tra_dtype dt, float sm_scale,
                                  hipStream_t s);

/*
 * Entropy -> budget -> radius -> block-sparse mask (Insight I: budget
 * tau * exp(H_i) / N; Insight II: the budget becomes a query-specific base
 * radius scaled per frame by phi(delta) = exp(-gamma * delta); pipeline
 * steps 2-3: a 2D disk per frame, then a fused kernel doing distance
 * computation, radius comparison, block pruning and token voting).
 *
 * Definition computed (bit-exact, no transcendental evaluated on the device):
 * query i (tile-major position, frame f_i, spatial h_i, w_i) keeps key j iff
 * d2 = (h_i - h_j)^2 + (w_i - w_j)^2 is 0, or
 *      ln(d2) <= (double)H_i + lambda[f_i][f_j],
 *      lambda[f][f'] = (ln tau - (2 gamma)|f - f'|) - ln(pi * S_f),
 *      S_f = sum_{f'=0}^{F-1} exp(-2 gamma |f - f'|),
 * with ln(d2) and lambda built in fp64 on the host with the C library.  This
 * is the disk d2 <= (r_i exp(-gamma |f_i - f_j|))^2 whose base radius r_i
 * makes the per-frame disk areas add up to the budget tau * exp(H_i).
 * Blocks are contiguous ranges of the tile-major sequence (block_q for
 * queries, block_k for keys; ragged last blocks).  votes(Qb, Kb) = number of
 * queries of Qb whose disk meets Kb; Kb is retained iff
 * votes >= vote_threshold or Kb overlaps Qb's own index range.
 *
 * entropy: device fp32 [outer][N], tile-major order (the warm-up entropies,
 * reused across later steps).  N = F*H*W.  tau > 0, gamma >= 0 (finite),
 * vote_threshold >= 1, block_q in {64, 128}, block_k = 64, tile >= 1.
 * Outputs (device):
 *   kv_count [outer][nqb]          number of retained k-blocks per q-block
 *   kv_index [outer][nqb][nkb]     ascending retained k-block indices, row
 *                                  stride nkb = ceil(N / block_k); entries
 *                                  past kv_count are unspecified
 *   block_mask [outer][nqb][nkb]   optional (may be NULL): 1 = retained
 * kv_index_capacity is the number of int32 elements of kv_index; fewer than
 * outer*nqb*nkb returns TRA_ERR_CAPACITY.  The first call for a geometry
 * uploads tables synchronously (see tra_mask_prepare).
 */
tra_status tra_build_block_mask(const float *entropy, int outer, int F, int H, int W, float tau, float gamma,
                                int block_q, int block_k, int vote_threshold, int tile_h, int tile_w,
                                int32_t *kv_count, int32_t *kv_index, int64_t kv_index_capacity,
                                uint8_t *block_mask, hipStream_t s);

/* Builds and uploads, on the current device (blocking), the tables that
 * tra_build_block_mask and tra_dense_attn_entropy_mask need for this geometry,
 * and the band table and compute-unit count that tra_sparse_schedule needs for
 * it and block_q, so that those calls do no allocation or upload later. */
tra_status tra_mask_prepare(int F, int H, int W, float tau, float gamma, int block_q, int block_k, int tile_h,
                            int tile_w);

/*
 * The 1D-distance variant of the mask (section 4, ablation study: the radius
 * mask replaced by a 1D distance), in the same block-sparse format.
 *
 * Definition computed (bit-exact, no transcendental evaluated on the device):
 * query i (tile-major position; natural raster index n_i = (f*H + h)*W + w)
 * keeps key j iff d = |n_i - n_j| is 0 or
 *      ln(d) <= (double)H_i + mu,   mu = ln tau - ln 2,
 * with ln(d) and mu built in fp64 on the host with the C library: the budget
 * tau * exp(H_i) of Insight I spent on a window of the flattened sequence
 * centred on the query, 2 d <= tau * exp(H_i).  No per-frame factor (the
 * sequence has no frame axis).  Blocks, votes, the diagonal rule and the
 * outputs are those of tra_build_block_mask.
 *
 * entropy: device fp32 [outer][N], tile-major.  N = F*H*W.  tau > 0 (finite),
 * vote_threshold >= 1, block_q in {64, 128}, block_k = 64, tile >= 1.  The
 * first call for a geometry and tau uploads tables (ln t for t < N, the
 * k-blocks' rectangles and natural-index bounds) synchronously
 * (tra_mask_prepare_1d does that ahead of time).
 */
tra_status tra_build_block_mask_1d(const float *entropy, int outer, int F, int H, int W, float tau, int block_q,
                                   int block_k, int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                   int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                   hipStream_t s);
/* Builds and uploads, on the current device (blocking), the tables of tra_build_block_mask_1d for
 * this geometry and tau, and the band table and compute-unit count of tra_sparse_schedule for it
 * and block_q.  Arguments and errors as tra_build_block_mask_1d's. */
tra_status tra_mask_prepare_1d(int F, int H, int W, float tau, int block_q, int block_k, int tile_h, int tile_w);

/*
 * Block-sparse attention over a kept mask (pipeline step 3: the regular
 * block-sparse mask runs on a block-sparse attention backend; cross-step
 * reuse: the mask from the warm-up entropies serves later denoising steps).
 *
 *   o_i = sum_{j in retained blocks of q-block(i)} softmax_j(sm_scale <q_i,k_j>) v_j
 *
 * over every token of each retained k-block, nothing else.  q, k, v, o as in
 * tra_dense_attn_entropy (tile-major order); kv_count / kv_index as written
 * by tra_build_block_mask for the same N, block_q, block_k (indices must be
 * in [0, nkb), ascending, counts in [1, nkb]; a row with count 0 yields zeros
 * and lse -inf.  Other values are clamped into those ranges, so every access
 * stays inside q, k, v and the list row, but the result is then unspecified).
 * lse: optional fp32 [outer][N].  With every block retained the result equals
 * tra_dense_attn_entropy's bit for bit (same tile order, same arithmetic).
 * bf16: each head's K and V are read as raw buffers, so N * D * 2 must stay
 * below 2^31 bytes (N < 8,388,608 at D = 128); larger returns
 * TRA_ERR_UNSUPPORTED before any HIP call.
 */
tra_status tra_block_sparse_attn(const void *q, const void *k, const void *v, void *o, float *lse,
                                 const int32_t *kv_count, const int32_t *kv_index, int outer, int N, int D,
                                 tra_dtype dt, float sm_scale, int block_q, int block_k, hipStream_t s);

/*
 * Block-sparse attention with fp8 queries and keys (section 5: TRA is
 * complementary to quantization; the reused block-sparse mask of pipeline
 * step 3 applied to fp8 inputs).  The same result definition as
 * tra_block_sparse_attn, with the scores taken from fp8 q and k:
 *
 *   o_i = sum_{j in retained blocks of q-block(i)} softmax_j(sm_scale <q_i,k_j>) v_j
 *
 * q, k: device, [outer][N][D] fp8 in the OCP E4M3 format (one byte per
 * element: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F and
 * 0xFF are NaN; no infinities), TILE-MAJOR order.  The scores are computed
 * on the fp8 matrix cores with fp32 accumulation (the products of two E4M3
 * values are exact in fp32).  Any quantization scale belongs in sm_scale.
 * v, o: device, [outer][N][D] bf16.  lse: optional fp32 [outer][N].
 * kv_count / kv_index as for tra_block_sparse_attn (clamped the same way);
 * order: NULL, or a schedule from tra_sparse_schedule (as in
 * tra_block_sparse_attn_scheduled).
 * Supported: D = 128, block_q = 128, block_k = 64, N * D * 2 < 2^31 (as for
 * the bf16 call); anything else returns TRA_ERR_UNSUPPORTED before any HIP call.
 */
tra_status tra_block_sparse_attn_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                                     const int32_t *kv_count, const int32_t *kv_index, const int32_t *order,
                                     int outer, int N, int D, float sm_scale, int block_q, int block_k,
                                     hipStream_t s);

/*
 * The order in which the block-sparse calls take the (head, q-block) rows
 * (section 4: 9-19% of the interactions are kept, and the per-query budgets
 * differ by orders of magnitude, so the rows' k-block lists -- their work --
 * differ in length).  Writes order[outer * nqb], a permutation of the rows
 * o * nqb + qb, for tra_block_sparse_attn_scheduled and
 * tra_block_sparse_attn_fp8, computed once per mask like kv_index:
 *  - when the grid is fewer than 2 waves of resident workgroups (two per
 *    compute unit): longest first, rows sorted by kv_count, largest first,
 *    ties by row (a list-scheduling order: the shortest rows end the grid);
 *  - otherwise: the spatial band order, within each head the q-blocks sorted
 *    by (row of tiles, frame, position along the row of tiles) of their
 *    centre token, dealt to the 8 XCDs in runs of 64 rows, so that the rows an
 *    XCD holds at once share most of their k-blocks in its L2.
 * Either way results are those of tra_block_sparse_attn bit for bit; only the
 * time changes.  kv_count: device int32 [outer][nqb] (read for the first
 * order); order: device int32, order_capacity elements (fewer than
 * outer * nqb returns TRA_ERR_CAPACITY).  block_q in {64, 128}, block_k = 64.
 * The first call for a geometry builds and uploads the band table
 * (nqb int32) synchronously; it stays in the per-device cache
 * (tra_mask_prepare and tra_mask_prepare_1d do that ahead of time).
 */
tra_status tra_sparse_schedule(const int32_t *kv_count, int outer, int F, int H, int W, int block_q, int block_k,
                               int tile_h, int tile_w, int32_t *order, int64_t order_capacity, hipStream_t s);

/*
 * tra_block_sparse_attn with workgroup b running the row order[b] (a schedule
 * written by tra_sparse_schedule for the same kv_count, outer, N, block_q).
 * Arguments and limits as tra_block_sparse_attn's; results equal it bit for
 * bit.  order must be a
 * permutation of [0, outer * nqb); other values are clamped into that range
 * (every access stays in bounds, but rows may then be left unwritten).
 */
tra_status tra_block_sparse_attn_scheduled(const void *q, const void *k, const void *v, void *o, float *lse,
                                           const int32_t *kv_count, const int32_t *kv_index, const int32_t *order,
                                           int outer, int N, int D, tra_dtype dt, float sm_scale, int block_q,
                                           int block_k, hipStream_t s);

/*
 * Warm-up pass with the mask fused in: tra_dense_attn_entropy followed by
 * tra_build_block_mask on its entropies, in one kernel ("Token Radius
 * Attention for Efficient Video Generation", section 2, TRA pipeline: the
 * entropy of step 1 feeds the radius mapping and the fused mask kernel of
 * steps 2-3; section 3, the entropy and mask kernels co-designed to keep the
 * overhead small).  A workgroup (two 128-query blocks) builds both q-blocks'
 * mask rows as soon as their entropies are final, in its own on-chip memory.
 *
 * Results equal those of the two separate calls bit for bit: o, entropy and
 * lse as tra_dense_attn_entropy writes them; kv_count, kv_index and
 * block_mask as tra_build_block_mask writes them from that entropy.
 * Arguments: as in those two calls, with N = F*H*W; entropy and lse may be
 * NULL (the mask still uses the entropies).  Supported: bf16, D = 128,
 * block_q = 128, block_k = 64, and geometries whose per-q-block mask state
 * fits the kernel's tile buffers (at most 64 frames); anything else returns
 * TRA_ERR_UNSUPPORTED before any HIP call.  The first call for a geometry
 * uploads the mask tables synchronously (see tra_mask_prepare).
 */
tra_status tra_dense_attn_entropy_mask(const void *q, const void *k, const void *v, void *o, float *entropy,
                                       float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                       float sm_scale, float tau, float gamma, int block_q, int block_k,
                                       int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                       int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                       hipStream_t s);

/*
 * The two attention passes on NATURAL-order tensors, with the tile-major
 * permutation folded into their loads and stores (pipeline step 3: the
 * tile-major layout keeps spatial neighbours contiguous; here it is applied
 * while the kernels copy rows, so no permuted copy of q, k, v or o exists).
 * o is written in natural order, while entropy and lse (each may be NULL)
 * stay indexed by TILE-MAJOR position, the order tra_build_block_mask reads,
 * and kv_count / kv_index are the tile-major block lists it writes.
 *
 * The sparse call equals, bit for bit,
 *   tra_tile_major_permute of q, k, v; tra_block_sparse_attn; and
 *   tra_tile_major_unpermute of o,
 * for the same tile_h, tile_w.  The dense calls (below and the fused one) see
 * every key, so they read k and v as they lie and sum over the keys in natural
 * order: they equal, bit for bit, the tile-major call on permuted q with k
 * and v unpermuted, o unpermuted; against the fully permuted chain only the
 * rounding order of those sums differs (the results agree within the
 * attention tolerances, not bit for bit, and a mask entry whose entropy sits
 * on a threshold may differ with it).
 *
 * q, k, v, o: device, [outer][N][128] bf16, natural order, N = F*H*W.  The
 * sparse call takes its rows in the spatial band order of tra_sparse_schedule
 * (the geometry is known here; the first call for a geometry uploads that
 * table too).
 * Supported: bf16, D = 128, W and tile_w multiples of 4 (then every aligned
 * group of four tile-major positions is a run of four natural rows), N*D*2 <
 * 2^31 (as tra_block_sparse_attn's bf16 limit); sparse: block_q = 128,
 * block_k = 64.  Anything else returns
 * TRA_ERR_UNSUPPORTED before any HIP call.  The first call for a geometry
 * builds and uploads the map (N/4 int32 natural row indices) synchronously
 * (tra_natural_prepare does that ahead of time); it stays in the per-device
 * cache until the process ends.
 */
/*
 * tra_dense_attn_entropy_mask on natural-order q, k, v, o (the warm-up step in one call):
 * results equal tra_dense_attn_entropy_mask on permuted q and natural-order k, v bit for bit,
 * with o unpermuted (the keys in natural order, as above); entropy, lse and the block lists
 * are tile-major, the lists those tra_build_block_mask writes from this call's entropies.
 * Supported: the intersection of what the two calls above support.
 */
tra_status tra_dense_attn_entropy_mask_natural(const void *q, const void *k, const void *v, void *o, float *entropy,
                                               float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                               float sm_scale, float tau, float gamma, int block_q, int block_k,
                                               int vote_threshold, int tile_h, int tile_w, int32_t *kv_count,
                                               int32_t *kv_index, int64_t kv_index_capacity, uint8_t *block_mask,
                                               hipStream_t s);
/* Builds and uploads the tile-major map and the band order (block_q = 128) the natural-order
 * calls use for this geometry on the current device (blocking), so that a timed or captured
 * call does no allocation or upload.  Returns
 * TRA_ERR_UNSUPPORTED for the geometries those calls reject (W or tile_w not a multiple of 4),
 * TRA_ERR_INVALID_ARG for non-positive sizes. */
tra_status tra_natural_prepare(int F, int H, int W, int tile_h, int tile_w);
tra_status tra_dense_attn_entropy_natural(const void *q, const void *k, const void *v, void *o, float *entropy,
                                          float *lse, int outer, int F, int H, int W, int D, tra_dtype dt,
                                          float sm_scale, int tile_h, int tile_w, hipStream_t s);
tra_status tra_block_sparse_attn_natural(const void *q, const void *k, const void *v, void *o, float *lse,
                                         const int32_t *kv_count, const int32_t *kv_index, int outer, int F, int H,
                                         int W, int D, tra_dtype dt, float sm_scale, int block_q, int block_k,
                                         int tile_h, int tile_w, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* TRA_H_ */
