// Tiled GEMM kernels for gfx950 (CDNA4): C[M,N] = A[M,K] @ B[K,N], fp16/bf16 in,
// fp32 accumulate, fp16/bf16/fp32 out.
//
// What is computed follows the naive tiled and naive persistent matmul listings
// of "(1/n) Triton matmul ... persistent kernel" (one output tile per program,
// fp32 accumulator reset per tile, masked loads that read zero outside M/N/K,
// masked store) and the merged loop of "(3/n) ... cross tile pipelining".  How
// it is computed is this file's own design for MI355X:
//
//  * A workgroup owns a BM x BN output tile and walks K in BK slices.  Each slice
//    of A (BM x BK) and B (BK x BN) is staged in LDS in a two-slot ring: while
//    the MFMAs consume slot s, the next slice is already in flight from global
//    memory into registers and lands in slot s^1 before the single barrier of
//    the step.
//  * Both operands sit in LDS "K-contiguous": A as [m][k] (its natural layout),
//    B transposed to [n][k] on the way in (each loader thread reads an 8x8 or 4x8
//    (k x n) block with 16-byte row loads and transposes it in registers with
//    byte permutes), so that every MFMA operand fragment is one 16-byte LDS read.
//    16-byte chunks of each LDS row are XOR-swizzled by the row index so that the
//    8 lanes served together by the LDS touch 8 different bank groups on both
//    the writes and the fragment reads.
//  * The product uses v_mfma_f32_32x32x16_{f16,bf16}.  The operands are fed as
//    (B fragment, A fragment), so each 32x32 accumulator block holds C^T: a lane
//    owns 4 consecutive columns of one row, and the epilogue writes 8- or
//    16-byte vectors.
//  * Waves are arranged WM x WN over the tile; wave (wm, wn) owns a (BM/WM) x
//    (BN/WN) sub-tile of FM x FN accumulator blocks.
//  * Tile order and the persistent / flattened loops come from schedule.hpp; the
//    trace kernel runs the same functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace ts {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct InF16 {};
struct InBF16 {};
struct OutF16 {};
struct OutBF16 {};
struct OutF32 {};

// Arguments of one GEMM launch (by value in the kernel argument segment).
struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int M, N, K;
    long long lda, ldb, ldc;  // row strides in elements (inner strides are 1)
    int vec_a, vec_b, vec_c;  // 1 if rows allow 16-byte (A, B) / full-width (C) vectors
    SchedArgs s;
};

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;             // threads
    static constexpr int TM = BM / WM, TN = BN / WN;    // wave sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 blocks per wave
    static constexpr int KCH = BK / 8;                  // 16-byte chunks per LDS row
    static constexpr int NA = BM * KCH;                 // A chunks per slice
    static constexpr int CA = (NA + NT - 1) / NT;       // A chunks per thread
    static constexpr int KBH = (BK * BN / 64 >= NT) ? 8 : 4;  // k rows of a B loader block
    static constexpr int NB = (BK / KBH) * (BN / 8);    // B loader blocks per slice
    static constexpr int CB = (NB + NT - 1) / NT;       // B blocks per thread
    static constexpr int SLOT = (BM + BN) * BK;         // halfwords per ring slot
    static constexpr int LDS_BYTES = 2 * SLOT * 2;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave sub-tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0 && (KCH & (KCH - 1)) == 0, "BK must be 16 * power of two");
    static_assert(BK % KBH == 0, "BK must be a multiple of the B block height");
};

// ---- small device helpers ------------------------------------------------------

__device__ __forceinline__ int swz(int row, int kch) { return (row ^ (row >> 3)) & (kch - 1); }

template <class TI>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<InF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<InBF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Output element conversion (round to nearest even) and stores of 4 consecutive
// columns; `full` = all 4 inside N with an aligned address.
template <class TO> struct Out;
template <> struct Out<OutF32> {
    typedef float T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, bool vec) {
        if (vec && valid >= 4) {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = v[e];
        }
    }
};
template <> struct Out<OutF16> {
    typedef _Float16 T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, bool vec) {
        _Float16 h[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        if (vec && valid >= 4) {
            u32x2 w;
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
            *reinterpret_cast<u32x2*>(p) = w;
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = h[e];
        }
    }
};
template <> struct Out<OutBF16> {
    typedef __bf16 T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, bool vec) {
        __bf16 h[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        if (vec && valid >= 4) {
            u32x2 w;
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
            *reinterpret_cast<u32x2*>(p) = w;
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = h[e];
        }
    }
};

// 8 consecutive 16-bit elements p[0..7], those at or past `valid` read as zero.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t* p, int valid, bool vec) {
    if (vec && valid >= 8) return *reinterpret_cast<const u32x4*>(p);
    uint32_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = (q < valid) ? (uint32_t)p[q] : 0u;
    u32x4 r;
    r[0] = e[0] | (e[1] << 16);
    r[1] = e[2] | (e[3] << 16);
    r[2] = e[4] | (e[5] << 16);
    r[3] = e[6] | (e[7] << 16);
    return r;
}

// ---- the tile engine -------------------------------------------------------------

template <class Cfg, class TI, class TO, bool MASKED>
struct Engine {
    static constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
    static constexpr int FM = Cfg::FM, FN = Cfg::FN, KCH = Cfg::KCH;
    static constexpr int CA = Cfg::CA, CB = Cfg::CB, KBH = Cfg::KBH;

    const GemmArgs& g;
    uint16_t* lds;     // ring of two slots: [A: BM x BK][B: BN x BK] each
    int tid, lane, wm, wn;

    u32x4 ra[CA];          // A slice in flight
    u32x4 rb[CB][KBH];     // B slice in flight (KBH rows of 8 columns per block)
    f32x16 acc[FM][FN];

    __device__ __forceinline__ Engine(const GemmArgs& g_, uint16_t* lds_) : g(g_), lds(lds_) {
        tid = threadIdx.x;
        lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        wm = wave / Cfg::WN;
        wn = wave % Cfg::WN;
    }

    __device__ __forceinline__ void zero_acc() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    // Global -> registers: slice k of tile (m0, n0).
    __device__ __forceinline__ void load_slice(int m0, int n0, int k) {
        const int k0 = k * BK;
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int idx = c * NT + tid;
            const int row = idx / KCH, kc = idx % KCH;
            const int gm = m0 + row, gk = k0 + kc * 8;
            const uint16_t* p = g.A + (long long)gm * g.lda + gk;
            if (!MASKED) {
                ra[c] = *reinterpret_cast<const u32x4*>(p);
            } else {
                const bool in = (Cfg::NA % NT == 0 || idx < Cfg::NA) && gm < g.M;
                ra[c] = in ? load8_masked(p, g.K - gk, g.vec_a) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int idx = c * NT + tid;
            const int nb = idx % (BN / 8), kb = idx / (BN / 8);
            const int gn = n0 + nb * 8, gk = k0 + kb * KBH;
            const bool blk = Cfg::NB % NT == 0 || idx < Cfg::NB;
#pragma unroll
            for (int r = 0; r < KBH; ++r) {
                const uint16_t* p = g.B + (long long)(gk + r) * g.ldb + gn;
                if (!MASKED) {
                    rb[c][r] = blk ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
                } else {
                    rb[c][r] = (blk && gk + r < g.K) ? load8_masked(p, g.N - gn, g.vec_b)
                                                     : u32x4{0, 0, 0, 0};
                }
            }
        }
    }

    // Registers -> LDS slot; B is transposed to [n][k] on the way.
    __device__ __forceinline__ void store_slice(int slot) {
        uint16_t* sa = lds + slot * Cfg::SLOT;
        uint16_t* sb = sa + BM * BK;
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int idx = c * NT + tid;
            if (Cfg::NA % NT == 0 || idx < Cfg::NA) {
                const int row = idx / KCH, kc = idx % KCH;
                *reinterpret_cast<u32x4*>(sa + row * BK + ((kc ^ swz(row, KCH)) * 8)) = ra[c];
            }
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int idx = c * NT + tid;
            if (!(Cfg::NB % NT == 0 || idx < Cfg::NB)) continue;
            const int nb = idx % (BN / 8), kb = idx / (BN / 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // column j of the block: element j of every loaded row
                const int d = j >> 1;
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const int n = nb * 8 + j;
                if (KBH == 8) {
                    u32x4 col;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        col[q] = __builtin_amdgcn_perm(rb[c][2 * q + 1][d], rb[c][2 * q][d], sel);
                    *reinterpret_cast<u32x4*>(sb + n * BK + ((kb ^ swz(n, KCH)) * 8)) = col;
                } else {
                    u32x2 col;
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        col[q] = __builtin_amdgcn_perm(rb[c][2 * q + 1][d], rb[c][2 * q][d], sel);
                    *reinterpret_cast<u32x2*>(sb + n * BK + (((kb >> 1) ^ swz(n, KCH)) * 8) + (kb & 1) * 4) = col;
                }
            }
        }
    }

    // MFMAs over one LDS slot.
    __device__ __forceinline__ void compute(int slot) {
        const uint16_t* sa = lds + slot * Cfg::SLOT;
        const uint16_t* sb = sa + BM * BK;
        const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int ch = 2 * s + hk;
            u32x4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * Cfg::TM + i * 32 + r32;
                af[i] = *reinterpret_cast<const u32x4*>(sa + row * BK + ((ch ^ swz(row, KCH)) * 8));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * Cfg::TN + j * 32 + r32;
                bf[j] = *reinterpret_cast<const u32x4*>(sb + row * BK + ((ch ^ swz(row, KCH)) * 8));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<TI>(bf[j], af[i], acc[i][j]);
        }
    }

    // Accumulators -> C (round to the output type), masked to M x N.
    __device__ __forceinline__ void store_tile(int m0, int n0) {
        typedef typename Out<TO>::T T;
        T* C = reinterpret_cast<T*>(g.C);
        const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * Cfg::TM + i * 32 + r32;
            if (MASKED && m >= g.M) continue;
            T* crow = C + (long long)m * g.ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * Cfg::TN + j * 32 + 8 * q + 4 * hk;
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                  acc[i][j][4 * q + 3]};
                    if (!MASKED) {
                        Out<TO>::store4(crow + n, v, 4, true);
                    } else {
                        const int valid = g.N - n;
                        if (valid > 0) Out<TO>::store4(crow + n, v, valid, g.vec_c);
                    }
                }
            }
        }
    }
};

// ---- kernels -------------------------------------------------------------------------

// Tiled and persistent modes: for each of the program's tiles, a full pipeline
// (prologue load, K loop with one slice in flight, epilogue).
template <class Cfg, class TI, class TO, bool MASKED, int MODE>
__global__ void __launch_bounds__(Cfg::NT) gemm_tiles_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::SLOT];
    Engine<Cfg, TI, TO, MASKED> e(g, lds);
    const ProgramWork w(g.s, blockIdx.x);
    const int ntiles = (MODE == MODE_TILED) ? 1 : w.ntiles;
    for (int i = 0; i < ntiles; ++i) {
        int tm, tn;
        tile_coords(g.s, w.tile_id(i), tm, tn);
        const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
        e.zero_acc();
        if (g.s.ks > 0) {
            e.load_slice(m0, n0, 0);
            e.store_slice(0);
            __syncthreads();
            for (int k = 0; k < g.s.ks; ++k) {
                const int cur = k & 1;
                const bool more = k + 1 < g.s.ks;
                if (more) e.load_slice(m0, n0, k + 1);
                e.compute(cur);
                if (more) e.store_slice(cur ^ 1);
                __syncthreads();
            }
        }
        e.store_tile(m0, n0);
    }
}

// Flattened cross-tile mode: one loop over (tile, k) items; the slice of item
// it+1 -- the first slice of the next tile when item it ends a tile -- is in
// flight while item it is multiplied and, at a tile's last K step, stored.
template <class Cfg, class TI, class TO, bool MASKED>
__global__ void __launch_bounds__(Cfg::NT) gemm_flat_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::SLOT];
    Engine<Cfg, TI, TO, MASKED> e(g, lds);
    const ProgramWork w(g.s, blockIdx.x);
    const int total = w.total_items();
    if (total == 0) return;
    FlatCursor cur(w);
    int tm, tn;
    tile_coords(g.s, cur.tile, tm, tn);
    e.load_slice(tm * Cfg::BM, tn * Cfg::BN, cur.k);
    e.store_slice(0);
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        const int slot = it & 1;
        if (cur.k == 0) e.zero_acc();
        FlatCursor nxt = cur;
        nxt.advance(w);
        int ntm = tm, ntn = tn;
        const bool more = it + 1 < total;
        if (more) {
            if (nxt.tile != cur.tile) tile_coords(g.s, nxt.tile, ntm, ntn);
            e.load_slice(ntm * Cfg::BM, ntn * Cfg::BN, nxt.k);
        }
        e.compute(slot);
        if (cur.last_k(w)) e.store_tile(tm * Cfg::BM, tn * Cfg::BN);
        if (more) e.store_slice(slot ^ 1);
        __syncthreads();
        cur = nxt;
        tm = ntm;
        tn = ntn;
    }
}

// Schedule trace: one thread per program, the same functions as above.
__global__ void trace_kernel(SchedArgs s, int mode, int max_items, int32_t* out);

}  // namespace ts
