// attention.hip -- dense warm-up attention with fused per-query entropy, and
// block-sparse attention over a kept mask, on CDNA4 matrix cores.
//
// "Token Radius Attention for Efficient Video Generation": section 1 (dense 3D
// self-attention over the N video tokens), TRA pipeline step 1 (each query's
// entropy taken during the dense warm-up), step 3 (the block-sparse mask runs on
// a block-sparse attention backend; the warm-up mask is reused by later steps) and
// section 3 contribution 3 (entropy fused into the attention kernel).
//
// Both modes share one tile engine.  A workgroup owns 32 * NW queries (NW
// wavefronts, 32 queries each) and walks 64-key tiles: every k-block in order
// (dense) or the k-blocks listed in kv_index (sparse).  Per tile, per wavefront:
//   S^T = K Q^T     (keys x queries) on MFMA, K from LDS, Q^T held in registers;
//   online softmax  in base 2 with a lazily refreshed running max (the max is only
//                   moved when a tile raises it by more than 2^8, so the O rescale
//                   is skipped on almost every tile);
//   entropy         one extra FMA per score: with x = s * sm_scale * log2 e,
//                   l = sum 2^(x - m), t = sum 2^(x - m) (x - m); a move of the
//                   max m -> m' maps (l, t) to (a l, a (t + (m - m') l)),
//                   a = 2^(m - m'); at the end H = ln 2 (log2 l - t / l) nats;
//   O^T += V^T P^T  on MFMA, V^T from LDS, P^T straight from the S^T registers.
// The transposed products keep every per-query statistic inside one lane (a lane
// owns one query and half of the keys of each tile), so only the tile max crosses
// lanes (one swap between the two lane halves).  K and V^T tiles are double
// buffered in LDS (one barrier per tile); the next tile's global loads are in
// flight while the current tile is computed.
//
// LDS layouts (16-byte granules, XOR-swizzled so that the MFMA operand reads and
// the staging writes are bank-conflict free):
//   K   [64 keys][D]  : 16-byte chunk c of key row r sits at chunk c ^ (r & 7).
//   V^T [D][64 keys]  : 8-byte chunk c (4 consecutive keys) of dim row n sits at
//                       chunk perm(c) ^ 2 * ((n ^ (n >> 3)) & 7), where perm swaps
//                       bits 0 and 1 of c so that the 8 keys one lane feeds to an
//                       MFMA (keys 4h..4h+3 and 8+4h..8+4h+3 of a 16-key step) are
//                       one 16-byte read.
#include "tra_internal.h"

#include <hip/hip_bf16.h>

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

// workgroup id -> logical (head, q-block) id such that each XCD (workgroups are
// dispatched round-robin over 8) receives one contiguous range of logical ids, so
// neighbouring q-blocks -- which read mostly the same k-blocks -- share an L2.
__device__ inline int xcd_remap(int bid, int total) {
    const int q = total >> 3, r = total & 7;
    const int x = bid & 7, k = bid >> 3;
    return x * q + min(x, r) + k;
}

__device__ inline float wave_swap_halves(float v) { return __shfl_xor(v, 32); }

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
    const float mt = fmaxf(mloc, wave_swap_halves(mloc)) * c;
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

template <int D>
struct Bf16Tile {
    static constexpr int KROW = D * 2;                // bytes per K row
    static constexpr int KBYTES = KT * KROW;          // K tile bytes
    static constexpr int VBYTES = D * KT * 2;         // V^T tile bytes
    static constexpr int BUF = KBYTES + VBYTES;
    static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
    static constexpr int KUNITS = KT * KCH;           // 16-byte K units per tile
    static constexpr int VUNITS = (KT / 4) * (D / 8); // (4 keys x 8 dims) V units per tile
};

template <int D, int NT>
struct Bf16Stage {
    static constexpr int KL = (Bf16Tile<D>::KUNITS + NT - 1) / NT;
    static constexpr int VL = (Bf16Tile<D>::VUNITS + NT - 1) / NT;
    u32x4_t k[KL];
    u32x4_t v[VL][4];
};

// global -> registers for one 64-key tile starting at key0 (keys >= N read as zero)
template <int D, int NT>
__device__ inline void bf16_load_tile(Bf16Stage<D, NT> &st, const __bf16 *__restrict__ kp,
                                      const __bf16 *__restrict__ vp, int key0, int N, int tid) {
    using T = Bf16Tile<D>;
#pragma unroll
    for (int i = 0; i < Bf16Stage<D, NT>::KL; ++i) {
        const int u = tid + i * NT;
        const int r = u / T::KCH, ch = u - r * T::KCH;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (u < T::KUNITS && key0 + r < N)
            val = *reinterpret_cast<const u32x4_t *>(kp + (int64_t)(key0 + r) * D + ch * 8);
        st.k[i] = val;
    }
#pragma unroll
    for (int i = 0; i < Bf16Stage<D, NT>::VL; ++i) {
        const int u = tid + i * NT;
        const int dg = u % (D / 8), kg = u / (D / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = key0 + kg * 4 + j;
            u32x4_t val = {0u, 0u, 0u, 0u};
            if (u < T::VUNITS && key < N)
                val = *reinterpret_cast<const u32x4_t *>(vp + (int64_t)key * D + dg * 8);
            st.v[i][j] = val;
        }
    }
}

__device__ inline int vt_chunk(int c, int n) {
    const int pc = (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1);
    return pc ^ (2 * ((n ^ (n >> 3)) & 7));
}

// registers -> LDS (K swizzled, V transposed + swizzled)
template <int D, int NT>
__device__ inline void bf16_store_tile(const Bf16Stage<D, NT> &st, char *buf, int tid) {
    using T = Bf16Tile<D>;
    char *ks = buf;
    char *vs = buf + T::KBYTES;
#pragma unroll
    for (int i = 0; i < Bf16Stage<D, NT>::KL; ++i) {
        const int u = tid + i * NT;
        if (u < T::KUNITS) {
            const int r = u / T::KCH, ch = u - r * T::KCH;
            *reinterpret_cast<u32x4_t *>(ks + r * T::KROW + ((ch ^ (r & 7)) << 4)) = st.k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < Bf16Stage<D, NT>::VL; ++i) {
        const int u = tid + i * NT;
        if (u < T::VUNITS) {
            const int dg = u % (D / 8), kg = u / (D / 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {  // dims 8dg + 2w, 8dg + 2w + 1
                const unsigned a0 = st.v[i][0][w], a1 = st.v[i][1][w], a2 = st.v[i][2][w], a3 = st.v[i][3][w];
                // even dim: low halves; odd dim: high halves
                u32x2_t ev, od;
                ev[0] = (a0 & 0xffffu) | (a1 << 16);
                ev[1] = (a2 & 0xffffu) | (a3 << 16);
                od[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                od[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                const int n0 = dg * 8 + 2 * w, n1 = n0 + 1;
                *reinterpret_cast<u32x2_t *>(vs + n0 * (KT * 2) + (vt_chunk(kg, n0) << 3)) = ev;
                *reinterpret_cast<u32x2_t *>(vs + n1 * (KT * 2) + (vt_chunk(kg, n1) << 3)) = od;
            }
        }
    }
}

// ----------------------------------------------------------------------------------
// bf16 kernel
// ----------------------------------------------------------------------------------
template <int D, int NW, bool SPARSE, bool ENT>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int NT = NW * 64;
    constexpr int BQ = NW * 32;
    using T = Bf16Tile<D>;
    __shared__ __attribute__((aligned(16))) char smem[2 * T::BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, ql = lane & 31;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int o = bid / a.nqb;
    const int qb = bid - o * a.nqb;
    const int N = a.N;
    const int64_t head = (int64_t)o * N * D;
    const __bf16 *qp = static_cast<const __bf16 *>(a.q) + head;
    const __bf16 *kp = static_cast<const __bf16 *>(a.k) + head;
    const __bf16 *vp = static_cast<const __bf16 *>(a.v) + head;
    const int qi = qb * BQ + wave * 32 + ql;

    // Q^T operand: lane holds query qi, dims 16 ks + 8 h .. + 8
    bf16x8_t qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (qi < N) val = *reinterpret_cast<const u32x4_t *>(qp + (int64_t)qi * D + ks * 16 + h * 8);
        qf[ks] = __builtin_bit_cast(bf16x8_t, val);
    }

    int ntiles;
    const int32_t *list = nullptr;
    if (SPARSE) {
        const int64_t row = (int64_t)o * a.nqb + qb;
        ntiles = min(max(a.kv_count[row], 0), a.nkb);
        list = a.kv_index + row * a.nkb;
    } else {
        ntiles = a.nkb;
    }
    auto tile_kb = [&](int it) -> int {
        if (SPARSE) {
            const int kb = list[it];
            return (kb >= 0 && kb < a.nkb) ? kb : -1;
        }
        return it;
    };

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    RowState st{kMasked, 0.f, 0.f};
    const float c = a.c;

    Bf16Stage<D, NT> stage;
    if (ntiles > 0) {
        const int kb0 = tile_kb(0);
        bf16_load_tile<D, NT>(stage, kp, vp, kb0 >= 0 ? kb0 * KT : N, N, tid);
        bf16_store_tile<D, NT>(stage, smem, tid);
        if (ntiles > 1) {
            const int kb1 = tile_kb(1);
            bf16_load_tile<D, NT>(stage, kp, vp, kb1 >= 0 ? kb1 * KT : N, N, tid);
        }
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        char *cur = smem + (it & 1) * T::BUF;
        if (it + 1 < ntiles) bf16_store_tile<D, NT>(stage, smem + ((it + 1) & 1) * T::BUF, tid);
        if (it + 2 < ntiles) {
            const int kb2 = tile_kb(it + 2);
            bf16_load_tile<D, NT>(stage, kp, vp, kb2 >= 0 ? kb2 * KT : N, N, tid);
        }
        const int kb = tile_kb(it);
        if (kb >= 0) {
            const char *ks = cur;
            const char *vs = cur + T::KBYTES;
            // S^T = K Q^T : two 32-key blocks
            f32x16_t s[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
                const int key = b * 32 + ql;
#pragma unroll
                for (int ks2 = 0; ks2 < D / 16; ++ks2) {
                    const int ch = 2 * ks2 + h;
                    const bf16x8_t av =
                        *reinterpret_cast<const bf16x8_t *>(ks + key * T::KROW + ((ch ^ (key & 7)) << 4));
                    s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks2], s[b], 0, 0, 0);
                }
            }
            // keys past N in the ragged last tile
            const int key0 = kb * KT;
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
            // P^T operand for 16-key step j: this lane's S^T entries 8 (j & 1) .. + 8 of block j >> 1
            bf16x8_t pf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    bf16x2_t pr = __builtin_convertvector(
                        (float __attribute__((ext_vector_type(2)))){s[j >> 1][8 * (j & 1) + e],
                                                                     s[j >> 1][8 * (j & 1) + e + 1]},
                        bf16x2_t);
                    pf[j][e] = pr[0];
                    pf[j][e + 1] = pr[1];
                }
            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int n = db * 32 + ql;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pos = vt_chunk(4 * j + h, n);  // pair (4j + 2h, +1) after the bit swap
                    const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(vs + n * (KT * 2) + (pos << 3));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[j], oacc[db], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // combine the two lane halves of each query and write out
    const float l = st.l + wave_swap_halves(st.l);
    const float t = ENT ? st.t + wave_swap_halves(st.t) : 0.f;
    if (qi < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        __bf16 *op = static_cast<__bf16 *>(a.o) + head + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x2_t lo = __builtin_convertvector(
                    (float __attribute__((ext_vector_type(2)))){oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv},
                    bf16x2_t);
                bf16x2_t hi = __builtin_convertvector(
                    (float __attribute__((ext_vector_type(2)))){oacc[db][4 * r4 + 2] * inv,
                                                                 oacc[db][4 * r4 + 3] * inv},
                    bf16x2_t);
                u32x2_t w;
                w[0] = __builtin_bit_cast(unsigned, lo);
                w[1] = __builtin_bit_cast(unsigned, hi);
                *reinterpret_cast<u32x2_t *>(op + db * 32 + 8 * r4 + 4 * h) = w;
            }
        if (h == 0) {
            const int64_t idx = (int64_t)o * N + qi;
            if (ENT && a.ent) a.ent[idx] = l > 0.f ? kLn2 * (__log2f(l) - t / l) : 0.f;
            if (a.lse) a.lse[idx] = l > 0.f ? kLn2 * (st.m + __log2f(l)) : -INFINITY;
        }
    }
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
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
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
        if (SPARSE) {
            kb = list[it];
            if (kb < 0 || kb >= a.nkb) continue;  // uniform across the workgroup
        }
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

    const float l = st.l + wave_swap_halves(st.l);
    const float t = ENT ? st.t + wave_swap_halves(st.t) : 0.f;
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

template <int D, int NW>
hipError_t launch_d(const AttnArgs &a, int dtype, bool sparse, hipStream_t s) {
    const unsigned blocks = (unsigned)((int64_t)a.outer * a.nqb);
    const bool ent = a.ent != nullptr;
    if (dtype == 1) {
        if (sparse)
            attn_bf16_kernel<D, NW, true, false><<<blocks, NW * 64, 0, s>>>(a);
        else if (ent)
            attn_bf16_kernel<D, NW, false, true><<<blocks, NW * 64, 0, s>>>(a);
        else
            attn_bf16_kernel<D, NW, false, false><<<blocks, NW * 64, 0, s>>>(a);
    } else {
        if (sparse)
            attn_f32_kernel<D, NW, true, false><<<blocks, NW * 64, 0, s>>>(a);
        else if (ent)
            attn_f32_kernel<D, NW, false, true><<<blocks, NW * 64, 0, s>>>(a);
        else
            attn_f32_kernel<D, NW, false, false><<<blocks, NW * 64, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int D, int dtype, int block_q, bool sparse, hipStream_t s) {
    if (block_q == 64) return D == 64 ? launch_d<64, 2>(a, dtype, sparse, s) : launch_d<128, 2>(a, dtype, sparse, s);
    return D == 64 ? launch_d<64, 4>(a, dtype, sparse, s) : launch_d<128, 4>(a, dtype, sparse, s);
}

}  // namespace tra
