// attention.hip -- dense warm-up attention with fused per-query entropy, and
// block-sparse attention over a kept mask, on CDNA4 matrix cores.
//
// "Token Radius Attention for Efficient Video Generation": section 1 (dense 3D
// self-attention over the N video tokens), TRA pipeline step 1 (each query's
// entropy taken during the dense warm-up), step 3 (the block-sparse mask runs on
// a block-sparse attention backend; the warm-up mask is reused by later steps) and
// section 3 contribution 3 (entropy fused into the attention kernel).
//
// Both modes share one tile engine (bf16 inputs, fp32 accumulation).  A workgroup owns
// one q-block (sparse; two for dense, 8 wavefronts, so each staged tile serves twice the
// queries); each wavefront owns 32 queries and walks 64-key tiles: every k-block in order
// (dense) or the k-blocks listed in kv_index (sparse).  Per tile and wavefront:
//   S^T = K Q^T      on MFMA (v_mfma_f32_32x32x16_bf16), K from LDS, Q^T in registers,
//                    so a lane owns one query and 32 of the tile's keys;
//   softmax          in base 2 with a lazily moved running max (it only moves when a
//                    tile raises it by more than 2^8, so O is rarely rescaled);
//   entropy          one extra FMA per score: with x = s * sm_scale * log2 e,
//                    l = sum 2^(x - m), t = sum 2^(x - m) (x - m); moving the max
//                    m -> m' maps (l, t) to (a l, a (t + (m - m') l)), a = 2^(m - m');
//                    at the end H = ln 2 (log2 l - t / l) nats;
//   O^T += V^T P^T   on MFMA, P^T straight from the S^T registers (bf16), the
//                    exponentials of one 16-key chunk running under the products of the
//                    previous chunk.
// Per-query statistics stay inside one lane; the two lanes that share a query combine
// with one v_permlane32_swap.  K and V tiles are copied global -> LDS directly (no
// staging registers) into double buffers while the current tile is computed; one
// barrier per tile.  Workgroups are ordered so that the 8 XCDs work through the same
// heads together, each on runs of neighbouring q-blocks.  The warm-up variant
// attn_mask_kernel ends with the mask builder (mask_impl.h) for its own q-block, run in
// the freed tile buffers (TRA pipeline steps 2-3 fused into the entropy pass).  The NAT
// instantiations read natural-order q, k, v and write natural-order o, with the
// tile-major map (pipeline step 3's layout) applied to the query and output rows, and in
// the sparse one to the K and V copies too (bit for bit the tile-major kernel on permuted
// tensors); the dense ones take K and V in natural order.
#include "mask_impl.h"
#include "tra_internal.h"

#include <hip/hip_bf16.h>

#include <type_traits>

namespace tra {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int KT = 64;              // keys per tile = block_k
constexpr float kMasked = -1.0e30f; // score of a key past N (finite: 0 * it stays 0)
constexpr float kLazy = 8.0f;       // max moves only when it grows by more than this (log2 units)
constexpr float kLn2 = 0.69314718055994530942f;

// workgroup id -> logical (head, q-block) id.  Workgroups are dispatched round-robin
// over the 8 XCDs; XCD x receives chunks of kXcdChunk consecutive logical ids (about
// the q-blocks it runs at once, so neighbouring q-blocks -- which read mostly the same
// k-blocks -- share its L2), and the chunks of the 8 XCDs advance together through the
// (head, q-block) order, so all XCDs stay in the same one or two heads and those heads'
// K and V stay within the last-level cache.  The ragged last row of chunks keeps the
// identity map (every id still appears exactly once).
constexpr int kXcdChunk = 32;
__device__ inline int xcd_remap(int bid, int total) {
    const int full = (total / (8 * kXcdChunk)) * (8 * kXcdChunk);
    if (bid >= full) return bid;
    const int x = bid & 7, k = bid >> 3;
    return (k / kXcdChunk) * (8 * kXcdChunk) + x * kXcdChunk + (k % kXcdChunk);
}

// The (head, q-block) row workgroup b runs: order[b] when the caller passes a schedule (clamped,
// so any value stays in bounds); else, with one head's band order, that order dealt to the XCDs in
// runs (the schedule's band order, computed here); else the XCD order above.
__device__ inline int row_of_workgroup(const AttnArgs &a, int b, int total) {
    typedef const int32_t __attribute__((address_space(4))) *cint_t;
    if (a.order) {
        const int r = ((cint_t)a.order)[b];
        return min(max(r, 0), total - 1);
    }
    if (a.band) {
        const int L = xcd_runs(b, total);
        const int o = L / a.nqb;
        return o * a.nqb + ((cint_t)a.band)[L - o * a.nqb];
    }
    return xcd_remap(b, total);
}

// Lane l and lane l ^ 32 hold the two halves of one query's keys.  v_permlane32_swap on two
// copies of v leaves {v[l], v[l ^ 32]} in the two results of every lane.  The results are
// copied to scalars before the bit cast: a bit cast applied directly to an element of the
// returned vector reads element 0 for both (a front-end code generation bug).
__device__ inline void pair_values(float v, float &a, float &b) {
#if defined(__HIP_DEVICE_COMPILE__)
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
#else
    a = v;
    b = v;
#endif
}
__device__ inline float pair_max(float v) {
    float a, b;
    pair_values(v, a, b);
    return fmaxf(a, b);
}
__device__ inline float pair_sum(float v) {
    float a, b;
    pair_values(v, a, b);
    return a + b;
}

// ----------------------------------------------------------------------------------
// softmax / entropy state of one lane (one query, half of each tile's keys)
// ----------------------------------------------------------------------------------
struct RowState {
    float m;  // running reference max, log2 units (x = s * c)
    float l;  // sum 2^(x - m) over this lane's keys
    float t;  // sum 2^(x - m) (x - m) over this lane's keys
};

template <bool ENT, int NACC>
__device__ inline void online_softmax(f32x16_t (&s)[2], RowState &st, float c, f32x16_t (&oacc)[NACC]) {
    float mloc = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[b][r]);
    const float mt = pair_max(mloc) * c;
    if (__any(mt > st.m + kLazy)) {
        const float mn = fmaxf(st.m, mt);
        const float al = __builtin_amdgcn_exp2f(st.m - mn);
        if (ENT) st.t = st.l > 0.f ? al * (st.t + (st.m - mn) * st.l) : 0.f;
        st.l *= al;
#pragma unroll
        for (int d = 0; d < NACC; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= al;
        st.m = mn;
    }
    const float nm = -st.m;
    float ls = 0.f, ts = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float d = fmaf(s[b][r], c, nm);
            const float e = __builtin_amdgcn_exp2f(d);
            ls += e;
            if (ENT) ts = fmaf(e, d, ts);
            s[b][r] = e;
        }
    st.l += ls;
    if (ENT) st.t += ts;
}

// ----------------------------------------------------------------------------------
// bf16 tile engine
//
// LDS holds K and V tiles row-major ([64 keys][D] bf16, no padding) in 16-byte chunks; chunk
// c of key row r is stored at chunk c ^ f(r).  The LDS of gfx950 serves 256 bytes (64 banks)
// per cycle, i.e. 16 lanes of a 16-byte read, and the swizzles make every operand read touch
// every 16-byte bank group the minimum number of times:
//   K (16-byte reads, 16 consecutive keys, same chunk):  f(r) = r & 15        (D = 128)
//                                                         f(r) = (r >> 1) & 7  (D = 64)
//   V (transpose reads, 8 rows x 64 contiguous bytes):   f(r) = 4 (r & 3)     (D = 128)
//                                                         f(r) = 4 ((r >> 1) & 1) (D = 64)
// Tiles arrive by direct global->LDS copies (each lane's 16 bytes land at base + 16 * lane,
// so a lane fetches the global chunk that belongs in its slot): no staging registers.
//  - K operand of S^T = K Q^T: lane (ql, h) reads key 32 b + ql, chunk 2 ks + h.
//  - V^T operand of O^T = V^T P^T: two LDS transpose reads (ds_read_b64_tr_b16) per MFMA.
//    Within each 16-lane group, output lane j receives element j % 4 of the 4-element rows
//    fetched by source lanes j / 4 + 4 k (k = 0..3); source lane 16 g + i points at key
//    16 s + 4 h + i / 4 (+ 8 for the second read), dims 32 db + 16 (g % 2) + 4 (i % 4), so
//    lane (ql, h) ends up with dim 32 db + ql of keys 16 s + 4 h + 0..3 and 16 s + 8 + 4 h +
//    0..3 -- exactly the keys whose probabilities it holds in its S^T registers.
// ----------------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

template <int D, int NT>
struct Bf16Cfg {
    static constexpr int ROW = D * 2;              // bytes per key row
    static constexpr int TILE = KT * ROW;          // bytes per K or V tile
    static constexpr int NCH = D / 8;              // 16-byte chunks per row
    static constexpr int SLOTS = KT * NCH;         // 16-byte slots per tile
    static constexpr int DMA = SLOTS / NT;         // slots per thread per tile
    static constexpr int LDS = 4 * TILE;           // K x2, V x2
    static_assert(SLOTS % NT == 0, "tile must split evenly over the workgroup");
    static __device__ inline int fK(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ inline int fV(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// v, hidden from the optimiser at this point: a value derived from it is computed here, not
// hoisted out of the loop into a register of its own.
__device__ inline int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// A uniform pointer, hidden from the optimiser: kept as the copy's scalar base rather than
// folded into a 64-bit vector address together with the lane offset.
__device__ inline const char *uniform_ptr(const char *p) {
    asm volatile("" : "+s"(p));
    return p;
}

// A copy's 32-bit lane offset, zero-extended.  The empty asm hides where the value comes
// from, so the compiler cannot fold the uniform table offset into a loop-invariant 64-bit
// vector address; the copy keeps the SGPR-base form: uniform base + this offset.
__device__ inline uint64_t lane_offset(int off) {
    asm volatile("" : "+v"(off));
    return (uint64_t)(uint32_t)off;
}

// lane i's value of v, uniform (the host pass of the compiler does not know the builtin)
__device__ inline int lane_value(int v, int i) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_readlane(v, i);
#else
    return v + 0 * i;
#endif
}

// Copy m of a tile moves its 64 slots 64 m .. 64 m + 63: rows m RPI .. m RPI + RPI - 1 (RPI =
// rows per copy).  The swizzles are XOR-linear in the row (f(m RPI + r) = f(m RPI) ^ f(r),
// r < RPI), so a lane's offset in copy m is its offset in copy 0, soff0, with the chunk bits
// flipped by copy_xor(m), plus m RPI rows (1024 bytes).
template <int D, int NT, bool ISV>
__device__ inline int copy_xor(int m) {
    using C = Bf16Cfg<D, NT>;
    constexpr int RPI = 64 / C::NCH;
    return (ISV ? C::fV(m * RPI) : C::fK(m * RPI)) << 4;
}

// direct global -> LDS copy of one full tile; src: the tile's first byte; the wavefront's
// copies are DMA consecutive ones starting at copy DMA * wave.
template <int D, int NT, bool ISV>
__device__ inline void dma_tile(const char *__restrict__ src, lds_char_t *dst, int soff0, int wave) {
    using C = Bf16Cfg<D, NT>;
    // a uniform base plus a zero-extended 32-bit lane offset selects the copy's SGPR-base form
    // (no 64-bit address arithmetic per copy), and a uniform wavefront index keeps the LDS
    // destination (M0) in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(wave);
    const int s0 = opaque(soff0);  // so that the per-copy offsets are not hoisted into registers
#pragma unroll
    for (int i = 0; i < C::DMA; ++i) {
        const int m = w * C::DMA + i;
        // the copy's rows as a uniform base (an LDS-DMA instruction offset would move the LDS
        // destination too), plus the lane offset
        __builtin_amdgcn_global_load_lds(uniform_ptr(src + m * 1024) + lane_offset(s0 ^ copy_xor<D, NT, ISV>(m)),
                                         dst + m * 1024, 16, 0, 0);
    }
}

// the same with a lane offset per copy (relative to src)
template <int NDMA>
__device__ inline void dma_tile_lanes(const char *__restrict__ src, lds_char_t *dst, const int *soff, int wave) {
    const int w = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
        __builtin_amdgcn_global_load_lds(src + (uint64_t)(uint32_t)soff[i], dst + (w * NDMA + i) * 1024, 16, 0, 0);
}

// Tile-major row p of a natural-order tensor is natural row nat4[p / 4] + p % 4: every
// aligned group of four tile-major rows is a run of four natural rows (the row of a tile
// whose width is a multiple of four).  Read through the constant address space, so a
// uniform index gives a scalar load.
typedef const int32_t __attribute__((address_space(4))) *nat_table_t;

__device__ inline int natural_row(nat_table_t nat4, int p) { return nat4[p >> 2] + (p & 3); }

// NAT: lane i < DMA of the result holds the byte offset (natural row * ROW) of row group
// w * DMA + i of the tile at key0, the groups this wavefront copies; read a step before the
// copy so that the copy never waits for the table (a vector load, retired with the copies of
// the step).
template <int D, int NT>
__device__ inline int nat_groups(const int32_t *__restrict__ nat4, int key0, int N, int wave, int lane) {
    using C = Bf16Cfg<D, NT>;
    return nat4[min((key0 >> 2) + wave * C::DMA + min(lane, C::DMA - 1), (N >> 2) - 1)] * C::ROW;
}

// copy the tile of 64 keys starting at (tile-major) key0; rows past N in a ragged last tile
// are fetched from row N - 1 (finite values; their scores are masked later).
// NAT (D = 128): base holds the rows in natural order.  A copy instruction moves four
// consecutive tile-major rows, one natural run; natv (nat_groups) holds the run's offset in
// lane i, and soff0 ^ copy_xor(m) is the lane's offset within the run (copy 0's rows are
// rows 0-3 of a run).  The ragged tile takes per-lane rows.
template <int D, int NT, bool ISV, bool NAT>
__device__ inline void fetch_tile(const char *__restrict__ base, nat_table_t nat4, int natv, int key0, int N,
                                  lds_char_t *dst, int soff0, int wave, int lane) {
    using C = Bf16Cfg<D, NT>;
    static_assert(!NAT || C::NCH == 16, "one copy instruction covers four rows only for D = 128");
    if (key0 + KT <= N) {
        if constexpr (NAT) {
            const int w = __builtin_amdgcn_readfirstlane(wave);
            const int s0 = opaque(soff0);
#pragma unroll
            for (int i = 0; i < C::DMA; ++i) {
                const int m = w * C::DMA + i;  // this copy's slots of the LDS tile
                const int off = lane_value(natv, i) + (s0 ^ copy_xor<D, NT, ISV>(m));
                __builtin_amdgcn_global_load_lds(base + lane_offset(off), dst + m * 1024, 16, 0, 0);
            }
        } else {
            dma_tile<D, NT, ISV>(base + (int64_t)key0 * C::ROW, dst, soff0, wave);
        }
    } else {
        // the ragged tile (once per workgroup at most): offsets computed here rather than kept
        // in registers across the loop
        const int ln = NAT ? lane : opaque(lane);
        int so[C::DMA];
#pragma unroll
        for (int i = 0; i < C::DMA; ++i) {
            const int sl = (wave * C::DMA + i) * 64 + ln;
            const int row = sl / C::NCH, p = sl % C::NCH;
            const int swz = (p ^ (ISV ? C::fV(row) : C::fK(row))) << 4;
            const int r = min(row, N - 1 - key0);
            so[i] = (NAT ? natural_row(nat4, key0 + r) : r) * C::ROW + swz;
        }
        dma_tile_lanes<C::DMA>(NAT ? base : base + (int64_t)key0 * C::ROW, dst, so, wave);
    }
}

struct NoCopies {
    __device__ inline void at(int) const {}
};

// The K and V tile copies of one step, issued between the S^T products (copy c after product
// c * NPOS / NC) instead of in one burst at the step's start: a burst holds the wavefront at
// the vector memory issue path while its matrix instructions wait.  Full tiles only.  The
// same copies as fetch_tile's: tile-major, ksrc / vsrc are the tiles' first bytes; NAT, they
// are the head's base and natK / natV hold the tiles' row groups (nat_groups).  K rows hold DK
// bf16 values' worth of bytes (DK = D/2 for fp8 keys), V rows D bf16 values; NPOS S^T products.
// BUF: the copies are buffer loads into LDS (MUBUF, the head's K and V as raw buffers, the tile's
// byte offset in soffset) instead of global_load_lds.  The global form is a FLAT instruction that
// the compiler's wait-count model takes for a possible LDS access completing out of order, so
// after one is issued every wait for an LDS operand becomes lgkmcnt(0) and drains all the K reads
// issued ahead of their products; with buffer loads each product waits for its own operand only.
template <int DK, int DV, int NT, bool NAT, int NPOS, bool BUF = false>
struct SpreadCopies {
    using CK = Bf16Cfg<DK, NT>;
    using CV = Bf16Cfg<DV, NT>;
    const char *ksrc, *vsrc;
    lds_char_t *kdst, *vdst;
    int soffK, soffV, natK, natV, w;
    __amdgpu_buffer_rsrc_t krs, vrs;  // BUF: the head's K and V as raw buffers
    int kbase, vbase;                 // BUF: byte offsets of the tiles in them

    template <bool ISV>
    __device__ inline void copy(int i) const {
        const int m = w * (ISV ? CV::DMA : CK::DMA) + i;
        const int so = ISV ? (soffV ^ copy_xor<DV, NT, true>(m)) : (soffK ^ copy_xor<DK, NT, false>(m));
        lds_char_t *dst = (ISV ? vdst : kdst) + m * 1024;
        if constexpr (NAT)
            __builtin_amdgcn_global_load_lds((ISV ? vsrc : ksrc) + lane_offset(lane_value(ISV ? natV : natK, i) + so), dst,
                                             16, 0, 0);
        else if constexpr (BUF)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ISV ? vrs : krs, dst, 16, so, (ISV ? vbase : kbase) + m * 1024, 0, 0);
        else
            __builtin_amdgcn_global_load_lds(uniform_ptr((ISV ? vsrc : ksrc) + m * 1024) + lane_offset(so), dst, 16, 0, 0);
    }
    __device__ inline void at(int n) const {
        constexpr int NC = CK::DMA + CV::DMA;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c * NPOS / NC == n) {
                if (c < CK::DMA)
                    copy<false>(c);
                else
                    copy<true>(c - CK::DMA);
            }
    }
};

// S^T = K Q^T for one 64-key tile and the wavefront's two 32-query blocks: each K operand
// read from LDS feeds two MFMAs (one per query block).  The two 32-key halves b are separate
// accumulation chains, issued alternately so that no product waits on the one before it (each
// chain still sums its products in the same order).  cp.at(n) runs after product n.
template <int D, int NT, int QW, class Copies = NoCopies>
__device__ inline void qk_tile(f32x16_t (&s)[2][QW], const lds_char_t *kb, const int (&koff)[D / 16],
                               const bf16x8_t (&qf)[QW][D / 16], const Copies &cp = Copies()) {
    using C = Bf16Cfg<D, NT>;
    const f32x16_t zero = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const bf16x8_t av =
                *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(kb + koff[ks] + b * 32 * C::ROW);
#pragma unroll
            for (int q2 = 0; q2 < QW; ++q2)
                s[b][q2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[q2][ks], ks == 0 ? zero : s[b][q2], 0, 0, 0);
            cp.at(2 * ks + b);
        }
    }
}

// S^T = K Q^T for one 64-key tile with fp8 (OCP e4m3) keys and queries on the fp8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4: the 64 products of a step reduce over 64 head dimensions).  LDS
// holds the K tile as rows of D bytes, 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7) (the
// layout of a 128-byte bf16 row).  Lane (ql, h) reads key 32 b + ql, dims 64 ks + 32 h .. + 32
// (chunks 4 ks + 2 h and 4 ks + 2 h + 1; koff8) and holds the same dims of its query (q8): A and B
// split the reduction the same way, so the product is the full dot product whatever order the
// matrix core takes the 32 bytes of a lane in.  cp.at(n) runs after product n.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int D, class Copies = NoCopies>
__device__ inline void qk_tile_f8(f32x16_t (&s)[2][1], const lds_char_t *kb, const int (&koff8)[D / 32],
                                  const i32x8_t (&q8)[D / 64], const Copies &cp = Copies()) {
    const f32x16_t zero = {};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
            typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
            const u32x4_t lo = *reinterpret_cast<lds_u32x4_t *>(kb + koff8[2 * ks] + b * 32 * D);
            const u32x4_t hi = *reinterpret_cast<lds_u32x4_t *>(kb + koff8[2 * ks + 1] + b * 32 * D);
            const i32x8_t av = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            // formats 0, 0: e4m3 for A and B; no block scales (the product is unscaled)
            s[b][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, q8[ks], ks == 0 ? zero : s[b][0], 0, 0, 0, 0,
                                                                      0, 0);
            cp.at(b * (D / 64) + ks);  // chains one after the other: measured faster here than alternated
        }
    }
}

template <int QW>
__device__ inline void mask_tail(f32x16_t (&s)[2][QW], int key0, int N, int h) {
    if (key0 + KT > N) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key0 + b * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= N) {
#pragma unroll
                    for (int q2 = 0; q2 < QW; ++q2) s[b][q2][r] = kMasked;
                }
    }
}

__device__ inline unsigned pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ inline void wait_dma() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's global->LDS copies have landed
}

// scaled max over this lane's 32 scores of query block q2, combined with the other half of
// the query's keys
template <int QW>
__device__ inline float tile_max(const f32x16_t (&s)[2][QW], int q2, float c) {
    float m = fmaxf(s[0][q2][0], s[1][q2][0]);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[b][q2][r]);
    return pair_max(m) * c;
}

// A workgroup of NW wavefronts owns 32 * QW * NW consecutive queries (one q-block); each
// wavefront owns QW 32-query MFMA blocks, so every K and V^T operand it reads from LDS feeds
// QW MFMAs.
//
// Step j (scores S_j already in registers, K_{j+1} and V_j in LDS; K_{j+2} and V_{j+1}
// copied in the background):
//   a. masking of keys past N (ragged last tile only); lazy max move for tile j
//   b. one basic block: P_j = exp2(S_j - m) and row sums (VALU), O^T += V^T_j P^T_j and
//      S^T_{j+1} = K_{j+1} Q^T (MFMA), so the exponentials run under both products
//   c. the max of tile j+1 (taken before its masking: keys past N are clamped duplicates
//      of a real key and cannot raise it)
//
// NAT: q, k, v and o are in natural token order; the entropy and lse stay indexed by
// tile-major position.  Queries and outputs go through the tile-major map (nat4).  The
// sparse kernel copies K and V through it too (NATKV: its block lists name tile-major
// k-blocks), so its arithmetic is that of the tile-major kernel on the permuted tensors, bit
// for bit.  A dense kernel sums over every key, in any order: the natural-order dense kernels
// take K and V as they lie, in natural row order, with the tile-major kernel's copies; only
// the rounding order of the sums differs from the tile-major kernel's.
// KF8: q and k are fp8 (OCP e4m3, one byte per element), S^T on the fp8 matrix cores (qk_tile_f8);
// v and o stay bf16 and everything after S^T is unchanged.  K rows are then D bytes: the tile
// configuration of a D/2-wide bf16 row (DK).
template <int D, int QW, bool KF8>
struct QRegs {
    bf16x8_t qf[QW][D / 16];  // lane holds queries q0 + 32 q2, dims 16 ks + 8 h .. + 8
};
template <int D, int QW>
struct QRegs<D, QW, true> {
    i32x8_t q8[D / 64];       // lane holds query q0, dims 64 ks + 32 h .. + 32 (fp8)
};

template <int D, int NW, int QW, bool SPARSE, bool ENT, bool NAT = false, bool KF8 = false>
struct Bf16Kernel {
    static constexpr int NT = NW * 64;
    static constexpr int DK = KF8 ? D / 2 : D;   // K row bytes / 2
    using C = Bf16Cfg<D, NT>;                   // V tiles (and K tiles unless KF8)
    using CK = Bf16Cfg<DK, NT>;                 // K tiles
    static_assert(!KF8 || (QW == 1 && !NAT && D == 128), "fp8 keys: one 32-query block per wavefront, D = 128");
    static constexpr int NPOS = KF8 ? 2 * (D / 64) : 2 * (D / 16);  // S^T products per tile
    // the tile-major sparse kernels issue their spread copies as buffer loads (the host keeps a
    // head's K and V under 2^31 bytes).  The dense kernels keep the global form: at the register
    // limit they run about 1% slower with it.  The natural-order sparse kernel keeps it too: its
    // per-lane row offsets gain nothing from the buffer form.
    static constexpr bool BUF = SPARSE && !NAT;
    static constexpr bool NATKV = NAT && SPARSE;  // K and V copied through the map
    using Spread = SpreadCopies<DK, D, NT, NATKV, NPOS, BUF>;

    struct Ctx {
        const char *kp, *vp;
        const int32_t __attribute__((address_space(4))) *list;
        nat_table_t nat4;
        const int32_t *nat4v;   // the same table, for vector loads
        int natK, natV;         // nat_groups of the tiles the next K and V copies fetch
        int keyV, keyK;         // fast sparse steps, tile-major: first keys of tiles j + 1, j + 2
        int N, nkb, nfull, ntiles, wave, lane, h;  // nfull: full 64-key tiles, N / 64
        float c;
        int koff[D / 16];  // K operand offsets (KF8: the first D / 32)
        int voff[D / 32];
        int soffK, soffV;  // lane offset in copy 0 of a K / V tile (copy_xor gives the others)
        __amdgpu_buffer_rsrc_t krs, vrs;  // BUF: the head's K and V
        QRegs<D, QW, KF8> qr;
        f32x16_t oacc[D / 32][QW];
        RowState st[QW];
        float mt[QW];  // scaled max of the tile whose scores are current
    };

    static __device__ inline int key0_of(const Ctx &x, int j) {
        if (SPARSE) return sparse_kblock(x.list[j], x.nkb) * KT;
        return j * KT;
    }
    // the same for the copies between the products, which move whole tiles: an entry naming
    // the ragged last k-block there (only an invalid list has one before its last entry) is
    // clamped to the last full one
    static __device__ inline int key0_full(const Ctx &x, int j) {
        if (SPARSE) return sparse_full_kblock(x.list[j], x.nfull) * KT;
        return j * KT;
    }

    // S^T of the tile in kb, with the copies of cp between the products (FAST) or none
    template <bool FAST>
    static __device__ inline void qk(const Ctx &x, f32x16_t (&sn)[2][QW], const lds_char_t *kb, const Spread &cp,
                                     std::integral_constant<bool, FAST>) {
        if constexpr (KF8) {
            const int(&k8)[D / 32] = *reinterpret_cast<const int(*)[D / 32]>(&x.koff[0]);
            if constexpr (FAST)
                qk_tile_f8<D>(sn, kb, k8, x.qr.q8, cp);
            else
                qk_tile_f8<D>(sn, kb, k8, x.qr.q8);
        } else {
            if constexpr (FAST)
                qk_tile<D, NT, QW>(sn, kb, x.koff, x.qr.qf, cp);
            else
                qk_tile<D, NT, QW>(sn, kb, x.koff, x.qr.qf);
        }
    }

    // kn: K_{j+1} (read); kd: buffer receiving K_{j+2}; vc: V_j (read); vd: buffer receiving
    // V_{j+1}; s: S_j; sn: receives S_{j+1} (computed unconditionally: past the last tile it
    // is unused).  Buffers are distinct LDS objects fixed at compile time, so the reads never
    // wait for the copies in flight.
    // FAST (j + 3 < ntiles: tiles j + 1 and j + 2 exist and are full, tile j is not the last):
    // the copies run between the S^T products, and (tile-major) the list entries come a step
    // ahead in keyV / keyK.  Otherwise the copies are issued at the step's start.
    template <bool FAST>
    static __device__ inline void step(Ctx &x, int j, lds_char_t *kn, lds_char_t *kd, lds_char_t *vc,
                                       lds_char_t *vd, f32x16_t (&s)[2][QW], f32x16_t (&sn)[2][QW]) {
        int natn = 0;  // NATKV: groups of tile j + 3, the K copy of the next step
        if constexpr (NATKV) natn = nat_groups<D, NT>(x.nat4v, key0_full(x, min(j + 3, x.ntiles - 1)), x.N, x.wave, x.lane);
        Spread cp{};
        if constexpr (FAST) {
            const int w = __builtin_amdgcn_readfirstlane(x.wave);
            if constexpr (NATKV)
                cp = Spread{x.kp, x.vp, kd, vd, opaque(x.soffK), opaque(x.soffV), x.natK, x.natV, w};
            else if constexpr (BUF)
                cp = Spread{nullptr, nullptr, kd, vd, opaque(x.soffK), opaque(x.soffV), 0, 0, w, x.krs, x.vrs,
                            (SPARSE ? x.keyK : key0_full(x, j + 2)) * CK::ROW,
                            (SPARSE ? x.keyV : key0_full(x, j + 1)) * C::ROW};
            else
                cp = Spread{x.kp + (int64_t)(SPARSE ? x.keyK : key0_full(x, j + 2)) * CK::ROW,
                            x.vp + (int64_t)(SPARSE ? x.keyV : key0_full(x, j + 1)) * C::ROW, kd, vd,
                            opaque(x.soffK), opaque(x.soffV), 0, 0, w};
        } else {
            if (j + 2 < x.ntiles)
                fetch_tile<DK, NT, false, NATKV>(x.kp, x.nat4, x.natK, key0_of(x, j + 2), x.N, kd, x.soffK, x.wave, x.lane);
            if (j + 1 < x.ntiles)
                fetch_tile<D, NT, true, NATKV>(x.vp, x.nat4, x.natV, key0_of(x, j + 1), x.N, vd, x.soffV, x.wave, x.lane);
        }

        // a.
        if constexpr (!FAST) mask_tail<QW>(s, key0_of(x, j), x.N, x.h);
        bool move = false;
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) move |= x.mt[q2] > x.st[q2].m + kLazy;
        if (__any(move)) {
#pragma unroll
            for (int q2 = 0; q2 < QW; ++q2) {
                const float mn = fmaxf(x.st[q2].m, x.mt[q2]);
                const float al = __builtin_amdgcn_exp2f(x.st[q2].m - mn);
                if (ENT) x.st[q2].t = x.st[q2].l > 0.f ? al * (x.st[q2].t + (x.st[q2].m - mn) * x.st[q2].l) : 0.f;
                x.st[q2].l *= al;
                x.st[q2].m = mn;
#pragma unroll
                for (int d = 0; d < D / 32; ++d)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x.oacc[d][q2][r] *= al;
            }
        }
        // b.
        const float c = x.c;
        // LLVM's small-GEMM interleave for this block: each matrix instruction followed by two
        // LDS reads, so the K operands are read ahead of their products (measured: 3% faster
        // sparse, dense and fused calls than the default schedule)
        __builtin_amdgcn_iglp_opt(0);
        qk(x, sn, kn, cp, std::integral_constant<bool, FAST>());
        float nm[QW], ls[QW], ts[QW];
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) {
            nm[q2] = -x.st[q2].m;
            ls[q2] = 0.f;
            ts[q2] = 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            u32x4_t pw[QW];
#pragma unroll
            for (int q2 = 0; q2 < QW; ++q2) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int b = jj >> 1, r = 8 * (jj & 1) + e;
                    const float d0 = fmaf(s[b][q2][r], c, nm[q2]), d1 = fmaf(s[b][q2][r + 1], c, nm[q2]);
                    const float e0 = __builtin_amdgcn_exp2f(d0), e1 = __builtin_amdgcn_exp2f(d1);
                    ls[q2] += e0 + e1;
                    if (ENT) ts[q2] = fmaf(e1, d1, fmaf(e0, d0, ts[q2]));
                    pw[q2][e >> 1] = pack_bf16x2(e0, e1);
                }
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const lds_char_t *src = vc + x.voff[db] + 16 * jj * C::ROW;
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)src);
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(src + 8 * C::ROW));
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int q2 = 0; q2 < QW; ++q2)
                    x.oacc[db][q2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, pw[q2]),
                                                                          x.oacc[db][q2], 0, 0, 0);
            }
        }
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) {
            x.st[q2].l += ls[q2];
            if (ENT) x.st[q2].t += ts[q2];
            // c.
            x.mt[q2] = tile_max<QW>(sn, q2, c);
        }
        if constexpr (NATKV) {
            x.natV = x.natK;
            x.natK = natn;
        }
        if constexpr (FAST) {
            if constexpr (SPARSE && !NAT) {
                // the list entry of tile j + 3 (< ntiles), read while this step's copies land
                __builtin_amdgcn_sched_barrier(0);
                x.keyV = x.keyK;
                x.keyK = key0_full(x, j + 3);
            }
            // this step's copies have landed; every wavefront is done reading (each LDS read
            // of the step has been consumed by its product, and the compiler may not move LDS
            // accesses across the barrier)
            wait_dma();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the list entry has arrived
        } else {
            // this step's copies have landed and every wavefront is done reading
            wait_dma();
            __syncthreads();
        }
    }

    // Epi: called once the outputs are written, with the four (now free) LDS tile buffers,
    // the (head, q-block), and this lane's query index, entropy and whether it exists; the
    // default does nothing.
    struct NoEpilogue {
        __device__ void operator()(lds_char_t *, lds_char_t *, lds_char_t *, lds_char_t *, int, int, int, float,
                                   bool) const {}
    };

    template <class Epi = NoEpilogue>
    static __device__ void run(const AttnArgs &a, const Epi &epi = Epi()) {
        constexpr int BQ = NW * 32 * QW;
        __shared__ __attribute__((aligned(1024))) char k0_raw[CK::TILE];
        __shared__ __attribute__((aligned(1024))) char k1_raw[CK::TILE];
        __shared__ __attribute__((aligned(1024))) char v0_raw[C::TILE];
        __shared__ __attribute__((aligned(1024))) char v1_raw[C::TILE];
        lds_char_t *K0 = (lds_char_t *)k0_raw, *K1 = (lds_char_t *)k1_raw;
        lds_char_t *V0 = (lds_char_t *)v0_raw, *V1 = (lds_char_t *)v1_raw;

        Ctx x;
        const int tid = threadIdx.x;
        x.lane = tid & 63;
        x.wave = tid >> 6;
        x.h = x.lane >> 5;
        const int ql = x.lane & 31, h = x.h, lane = x.lane;
        const int bid = row_of_workgroup(a, blockIdx.x, gridDim.x);
        const int o = bid / a.nqb;
        const int qb = bid - o * a.nqb;
        const int N = a.N;
        x.N = N;
        x.nkb = a.nkb;
        x.nfull = N / KT;
        x.c = a.c;
        const int64_t head = (int64_t)o * N * D;
        const __bf16 *qp = static_cast<const __bf16 *>(a.q) + head;
        // K rows are CK::ROW bytes (D bytes for fp8 keys)
        x.kp = static_cast<const char *>(a.k) + head * (CK::ROW / D);
        x.vp = reinterpret_cast<const char *>(static_cast<const __bf16 *>(a.v) + head);
        if constexpr (BUF) {
            // raw buffers over this head's K and V (word 3 for the gfx9 family: 32-bit data format,
            // no swizzle); num_records = the head's bytes, so the hardware also drops any access past them
            x.krs = __builtin_amdgcn_make_buffer_rsrc((void *)x.kp, (short)0, N * CK::ROW, 0x00020000);
            x.vrs = __builtin_amdgcn_make_buffer_rsrc((void *)x.vp, (short)0, N * C::ROW, 0x00020000);
        }
        const int q0 = qb * BQ + x.wave * 32 * QW + ql;  // query of block 0 (block q2: + 32 q2)

        x.natK = x.natV = 0;
        if constexpr (NAT) {
            x.nat4 = (nat_table_t)a.nat4;
            x.nat4v = a.nat4;
        } else {
            x.nat4 = nullptr;
            x.nat4v = nullptr;
        }
        // row of query q0 + 32 q2 in q and o (its tile-major position unless NAT)
        int qrow[QW];
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) {
            const int qi = q0 + 32 * q2;
            qrow[q2] = qi;
            if constexpr (NAT) qrow[q2] = qi < N ? natural_row(x.nat4, qi) : qi;
        }

        if constexpr (KF8) {
            // fp8 Q^T operands: lane holds query q0, dims 64 ks + 32 h .. + 32 (one byte each)
            const char *q8p = static_cast<const char *>(a.q) + head;
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks) {
                u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
                if (q0 < N) {
                    const char *src = q8p + (int64_t)qrow[0] * D + 64 * ks + 32 * h;
                    lo = *reinterpret_cast<const u32x4_t *>(src);
                    hi = *reinterpret_cast<const u32x4_t *>(src + 16);
                }
                x.qr.q8[ks] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            // K operand: chunks 4 ks + 2 h + part of key ql (+ 32 b), stored at chunk c ^ fK(ql)
            const int xk = CK::fK(ql);
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
                for (int part = 0; part < 2; ++part)
                    x.koff[2 * ks + part] = ql * CK::ROW + 16 * ((4 * ks + 2 * h + part) ^ xk);
        } else {
            // Q^T operands: lane holds queries q0 + 32 q2, dims 16 ks + 8 h .. + 8
#pragma unroll
            for (int q2 = 0; q2 < QW; ++q2) {
                const int qi = q0 + 32 * q2;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    u32x4_t val = {0u, 0u, 0u, 0u};
                    if (qi < N) val = *reinterpret_cast<const u32x4_t *>(qp + (int64_t)qrow[q2] * D + ks * 16 + h * 8);
                    x.qr.qf[q2][ks] = __builtin_bit_cast(bf16x8_t, val);
                }
            }
            // K operand: chunk 2 ks + h of key ql (+ 32 b), stored at chunk (2 ks + h) ^ fK(ql)
            const int xk = C::fK(ql);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                x.koff[ks] = ql * C::ROW + 32 * (ks ^ (xk >> 1)) + 16 * (h ^ (xk & 1));
        }
        {
            // V^T operand source: key 4 hh + i / 4 (+ 16 s, + 8), dims 32 db + 16 (g % 2) + 4 (i % 4)
            const int g = lane >> 4, i = lane & 15, hh = g >> 1;
            const int u = 2 * (g & 1) + ((i & 3) >> 1);
            const int row = 4 * hh + (i >> 2);
            const int sel = D == 128 ? (i >> 2) : ((i >> 3) & 1);  // fV(row) / 4
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                x.voff[db] = row * C::ROW + 64 * (db ^ sel) + 16 * u + 8 * (i & 1);
        }
        {
            // copy 0's slots: row lane / NCH, chunk lane % NCH; for NATKV the row counts within
            // the copy's run of four natural rows, which is the same number
            const int rk = lane / CK::NCH, pk = lane % CK::NCH;
            x.soffK = rk * CK::ROW + ((pk ^ CK::fK(rk)) << 4);
            const int row = lane / C::NCH, p = lane % C::NCH;
            x.soffV = row * C::ROW + ((p ^ C::fV(row)) << 4);
        }

        if (SPARSE) {
            const int64_t row = (int64_t)o * a.nqb + qb;
            x.ntiles = min(max(a.kv_count[row], 0), a.nkb);
            x.list = (const int32_t __attribute__((address_space(4))) *)(a.kv_index + row * a.nkb);
        } else {
            x.ntiles = a.nkb;
            x.list = nullptr;
        }
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) {
#pragma unroll
            for (int d = 0; d < D / 32; ++d) x.oacc[d][q2] = f32x16_t{};
            x.st[q2] = RowState{kMasked, 0.f, 0.f};
        }

        f32x16_t s0[2][QW], s1[2][QW];
        if (x.ntiles > 0) {
            const int k0 = key0_of(x, 0);
            int n0 = 0;
            if constexpr (NATKV) {
                n0 = nat_groups<D, NT>(x.nat4v, k0, N, x.wave, lane);
                x.natV = nat_groups<D, NT>(x.nat4v, key0_full(x, min(1, x.ntiles - 1)), N, x.wave, lane);
                x.natK = nat_groups<D, NT>(x.nat4v, key0_full(x, min(2, x.ntiles - 1)), N, x.wave, lane);
            }
            fetch_tile<DK, NT, false, NATKV>(x.kp, x.nat4, n0, k0, N, K0, x.soffK, x.wave, lane);
            fetch_tile<D, NT, true, NATKV>(x.vp, x.nat4, n0, k0, N, V0, x.soffV, x.wave, lane);
            if (x.ntiles > 1)
                fetch_tile<DK, NT, false, NATKV>(x.kp, x.nat4, x.natV, key0_of(x, 1), N, K1, x.soffK, x.wave, lane);
            wait_dma();
            __syncthreads();
            qk(x, s0, K0, Spread{}, std::integral_constant<bool, false>());
#pragma unroll
            for (int q2 = 0; q2 < QW; ++q2) x.mt[q2] = tile_max<QW>(s0, q2, x.c);
            __syncthreads();  // every wavefront is done with K_0 before K_2 overwrites it
            int j = 0;
            if constexpr (SPARSE && !NAT) {
                if (x.ntiles > 4) {
                    x.keyV = key0_full(x, 1);
                    x.keyK = key0_full(x, 2);
                }
            }
            // pairs of steps j, j + 1 with j + 4 < ntiles are fast (sparse_fast_steps)
            for (; j + 4 < x.ntiles; j += 2) {
                step<true>(x, j, K1, K0, V0, V1, s0, s1);
                step<true>(x, j + 1, K0, K1, V1, V0, s1, s0);
            }
            for (; j < x.ntiles; j += 2) {
                step<false>(x, j, K1, K0, V0, V1, s0, s1);
                if (j + 1 < x.ntiles) step<false>(x, j + 1, K0, K1, V1, V0, s1, s0);
            }
        }

        // combine the two lane halves of each query and write out
        float hq = 0.f;
#pragma unroll
        for (int q2 = 0; q2 < QW; ++q2) {
            const float l = pair_sum(x.st[q2].l);
            const float t = ENT ? pair_sum(x.st[q2].t) : 0.f;
            const int qi = q0 + 32 * q2;
            if (ENT) hq = l > 0.f ? kLn2 * (__log2f(l) - t / l) : 0.f;
            if (qi < N) {
                const float inv = l > 0.f ? 1.f / l : 0.f;
                __bf16 *op = static_cast<__bf16 *>(a.o) + head + (int64_t)qrow[q2] * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        u32x2_t w;
                        w[0] = pack_bf16x2(x.oacc[db][q2][4 * r4] * inv, x.oacc[db][q2][4 * r4 + 1] * inv);
                        w[1] = pack_bf16x2(x.oacc[db][q2][4 * r4 + 2] * inv, x.oacc[db][q2][4 * r4 + 3] * inv);
                        *reinterpret_cast<u32x2_t *>(op + db * 32 + 8 * r4 + 4 * h) = w;
                    }
                if (h == 0) {
                    const int64_t idx = (int64_t)o * N + qi;
                    if (ENT && a.ent) a.ent[idx] = hq;
                    if (a.lse) a.lse[idx] = l > 0.f ? kLn2 * (x.st[q2].m + __log2f(l)) : -INFINITY;
                }
            }
        }
        epi(K0, K1, V0, V1, o, qb, q0 - qb * BQ, hq, q0 < N && h == 0);
    }
};

// Mask epilogue of the fused warm-up kernel: each q-block's mask row is built as soon as its
// entropies are final, in the attention kernel's own LDS ("Token Radius Attention for
// Efficient Video Generation", section 2, TRA pipeline steps 2-3 fused with the entropy
// pass of step 1): no launch, and no entropy read back from HBM.  The workgroup holds two
// q-blocks (8 wavefronts, as the dense kernel): wavefronts 0-3 build the row of the first in
// the four freed tile buffers, wavefronts 4-7 the row of the second in four more, at once.
template <int RR>
struct MaskEpilogue {
    const MaskArgs *m;
    __device__ void operator()(lds_char_t *k0, lds_char_t *k1, lds_char_t *v0, lds_char_t *v1, int o, int qb, int qlocal,
                               float hq, bool valid) const {
        using namespace maskdev;
        __shared__ __attribute__((aligned(1024))) char e0[16384];
        __shared__ __attribute__((aligned(1024))) char e1[16384];
        __shared__ __attribute__((aligned(1024))) char e2[16384];
        __shared__ __attribute__((aligned(1024))) char e3[16384];
        __shared__ int visits[2];
        const int half = threadIdx.x >> 8;
        const int mqb = 2 * qb + half;
        void *b0 = half ? (void *)e0 : (void *)k0;
        void *b1 = half ? (void *)e1 : (void *)k1;
        void *b2 = half ? (void *)e2 : (void *)v1;
        void *b3 = half ? (void *)e3 : (void *)v0;
        const MaskLds<128, true> L(b0, b1, b2, b3, m->g.F, m->nqf_max);
        __syncthreads();  // every wavefront is past its last read of the tiles
        if (valid) L.H[qlocal & 127] = hq;
        mask_qblock<128, RR, true, true>(*m, L, o, mqb, threadIdx.x & 255, mqb < m->nqb, MaskPair{visits, half});
    }
};

// Two wavefronts per SIMD for the 4-wavefront workgroups (two workgroups per CU); the
// 8-wavefront ones get two per SIMD from a single workgroup, and the 2-wavefront ones
// (64-query blocks) are held to one per SIMD by their 64 KB of LDS anyway, so those
// two take the whole register file.
template <int D, int NW, int QW, bool SPARSE, bool ENT, bool NAT = false, bool KF8 = false>
__global__ __launch_bounds__(NW * 64, (QW == 1 && NW == 4) ? 2 : 1) void attn_bf16_kernel(AttnArgs a) {
    Bf16Kernel<D, NW, QW, SPARSE, ENT, NAT, KF8>::run(a);
}

// dense attention + entropy + the mask rows of two 128-query blocks per workgroup (D = 128,
// bf16; 128 KB of LDS, one workgroup per CU)
template <int RR, bool NAT>
__global__ __launch_bounds__(512, 1) void attn_mask_kernel(AttnArgs a, MaskArgs m) {
    Bf16Kernel<128, 8, 1, false, true, NAT>::run(a, MaskEpilogue<RR>{&m});
}

template <bool NAT>
hipError_t launch_dense_mask_t(const AttnArgs &b, const MaskArgs &m, unsigned blocks, hipStream_t s) {
    switch (m.t.rmax) {
        case 1: attn_mask_kernel<1, NAT><<<blocks, 512, 0, s>>>(b, m); break;
        case 2: attn_mask_kernel<2, NAT><<<blocks, 512, 0, s>>>(b, m); break;
        case 3: attn_mask_kernel<3, NAT><<<blocks, 512, 0, s>>>(b, m); break;
        case 4: attn_mask_kernel<4, NAT><<<blocks, 512, 0, s>>>(b, m); break;
        default: attn_mask_kernel<0, NAT><<<blocks, 512, 0, s>>>(b, m); break;
    }
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------
// fp32 kernel (fp32 matrix cores, v_mfma_f32_32x32x2f32): same structure, plain
// row-major LDS tiles padded by one float per row, P kept in fp32.
// ----------------------------------------------------------------------------------
template <int D, int NW, bool SPARSE, bool ENT>
__global__ __launch_bounds__(NW * 64, 1) void attn_f32_kernel(AttnArgs a) {
    constexpr int NT = NW * 64;
    constexpr int BQ = NW * 32;
    constexpr int LD = D + 1;  // padded row (floats)
    __shared__ float ksm[KT * LD];
    __shared__ float vsm[KT * LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, ql = lane & 31;
    const int bid = row_of_workgroup(a, blockIdx.x, gridDim.x);
    const int o = bid / a.nqb;
    const int qb = bid - o * a.nqb;
    const int N = a.N;
    const int64_t head = (int64_t)o * N * D;
    const float *qp = static_cast<const float *>(a.q) + head;
    const float *kp = static_cast<const float *>(a.k) + head;
    const float *vp = static_cast<const float *>(a.v) + head;
    const int qi = qb * BQ + wave * 32 + ql;

    float qf[D / 2];  // dims 2 ks + h
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qi < N ? qp[(int64_t)qi * D + 2 * ks + h] : 0.f;

    int ntiles;
    const int32_t *list = nullptr;
    if (SPARSE) {
        const int64_t row = (int64_t)o * a.nqb + qb;
        ntiles = min(max(a.kv_count[row], 0), a.nkb);
        list = a.kv_index + row * a.nkb;
    } else {
        ntiles = a.nkb;
    }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    RowState st{kMasked, 0.f, 0.f};
    const float c = a.c;

    for (int it = 0; it < ntiles; ++it) {
        int kb = it;
        if (SPARSE) kb = sparse_kblock(list[it], a.nkb);  // any entry stays inside k and v
        const int key0 = kb * KT;
        __syncthreads();
        for (int u = tid; u < KT * D; u += NT) {
            const int r = u / D, d = u - r * D;
            const bool ok = key0 + r < N;
            ksm[r * LD + d] = ok ? kp[(int64_t)(key0 + r) * D + d] : 0.f;
            vsm[r * LD + d] = ok ? vp[(int64_t)(key0 + r) * D + d] : 0.f;
        }
        __syncthreads();
        f32x16_t s[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
            const int key = b * 32 + ql;
#pragma unroll
            for (int ks = 0; ks < D / 2; ++ks)
                s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(ksm[key * LD + 2 * ks + h], qf[ks], s[b], 0, 0, 0);
        }
        if (key0 + KT > N) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + b * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (key >= N) s[b][r] = kMasked;
                }
        }
        online_softmax<ENT, D / 32>(s, st, c, oacc);
        // O^T += V^T P^T, one key pair (k-slots h) per MFMA step: this lane's S^T entry r
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int n = db * 32 + ql;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = b * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vsm[key * LD + n], s[b][r], oacc[db], 0, 0, 0);
                }
        }
    }

    const float l = pair_sum(st.l);
    const float t = ENT ? pair_sum(st.t) : 0.f;
    if (qi < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *op = static_cast<float *>(a.o) + head + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4 w = make_float4(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv, oacc[db][4 * r4 + 2] * inv,
                                       oacc[db][4 * r4 + 3] * inv);
                *reinterpret_cast<float4 *>(op + db * 32 + 8 * r4 + 4 * h) = w;
            }
        if (h == 0) {
            const int64_t idx = (int64_t)o * N + qi;
            if (ENT && a.ent) a.ent[idx] = l > 0.f ? kLn2 * (__log2f(l) - t / l) : 0.f;
            if (a.lse) a.lse[idx] = l > 0.f ? kLn2 * (st.m + __log2f(l)) : -INFINITY;
        }
    }
}

#ifndef TRA_BF16_QW
#define TRA_BF16_QW 1
#endif
constexpr int kQW = TRA_BF16_QW;  // 32-query MFMA blocks per wavefront in the bf16 kernels

template <int D, int NW, bool SPARSE, bool ENT>
hipError_t launch_bf16(const AttnArgs &a, unsigned blocks, hipStream_t s) {
    attn_bf16_kernel<D, NW, kQW, SPARSE, ENT><<<blocks, NW * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_d(const AttnArgs &a, int dtype, bool sparse, hipStream_t s) {
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    const bool ent = a.ent != nullptr;
    if (dtype == 1) {
        if (sparse) return launch_bf16<D, NW, true, false>(a, blocks, s);
        if (ent) return launch_bf16<D, NW, false, true>(a, blocks, s);
        return launch_bf16<D, NW, false, false>(a, blocks, s);
    } else if constexpr (NW <= 4) {  // the fp32 kernels run 2 or 4 wavefronts
        if (sparse)
            attn_f32_kernel<D, NW, true, false><<<blocks, NW * 64, 0, s>>>(a);
        else if (ent)
            attn_f32_kernel<D, NW, false, true><<<blocks, NW * 64, 0, s>>>(a);
        else
            attn_f32_kernel<D, NW, false, false><<<blocks, NW * 64, 0, s>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_mask(const AttnArgs &a, const MaskArgs &m, hipStream_t s) {
    AttnArgs b = a;
    b.nqb = (a.N + 255) / 256;  // attention blocks of two mask q-blocks
    const unsigned blocks = (unsigned)((int64_t)b.outer * b.nqb);
    return a.nat4 ? launch_dense_mask_t<true>(b, m, blocks, s) : launch_dense_mask_t<false>(b, m, blocks, s);
}

hipError_t launch_attention_fp8(const AttnArgs &a, hipStream_t s) {
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    attn_bf16_kernel<128, 4, 1, true, false, false, true><<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_attention_natural(const AttnArgs &a, bool sparse, hipStream_t s) {
    if (sparse) {
        const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
        attn_bf16_kernel<128, 4, 1, true, false, true><<<blocks, 256, 0, s>>>(a);
    } else {
        // as the tile-major dense kernels: 8 wavefronts, 256 queries per workgroup
        AttnArgs b = a;
        b.nqb = (a.N + 255) / 256;
        const unsigned blocks = (unsigned)((int64_t)b.outer * b.nqb);
        if (a.ent)
            attn_bf16_kernel<128, 8, 1, false, true, true><<<blocks, 512, 0, s>>>(b);
        else
            attn_bf16_kernel<128, 8, 1, false, false, true><<<blocks, 512, 0, s>>>(b);
    }
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int D, int dtype, int block_q, bool sparse, hipStream_t s) {
    // bf16: 32 * kQW queries per wavefront; fp32: 32 queries per wavefront
    if (dtype == 1) {
        constexpr int w64 = 2 / kQW, w128 = 4 / kQW;
        if (!sparse && kQW == 1) {
            // dense: every query block reads the same K/V tiles, so one workgroup of 8
            // wavefronts (256 queries, one per CU, still two wavefronts per SIMD) stages each tile
            // once for twice the queries: half the copy traffic per product
            AttnArgs b = a;
            b.nqb = (a.N + 255) / 256;
            return D == 64 ? launch_d<64, 8>(b, dtype, false, s) : launch_d<128, 8>(b, dtype, false, s);
        }
        if (block_q == 64) return D == 64 ? launch_d<64, w64>(a, dtype, sparse, s) : launch_d<128, w64>(a, dtype, sparse, s);
        return D == 64 ? launch_d<64, w128>(a, dtype, sparse, s) : launch_d<128, w128>(a, dtype, sparse, s);
    }
    if (block_q == 64) return D == 64 ? launch_d<64, 2>(a, dtype, sparse, s) : launch_d<128, 2>(a, dtype, sparse, s);
    return D == 64 ? launch_d<64, 4>(a, dtype, sparse, s) : launch_d<128, 4>(a, dtype, sparse, s);
}

}  // namespace tra
