// Tiled GEMM kernels for gfx950 (CDNA4): C[M,N] = A[M,K] @ B[K,N], fp16/bf16 in,
// fp32 accumulate, fp16/bf16/fp32 out.
//
// What is computed follows the naive tiled and naive persistent matmul listings
// of "(1/n) Triton matmul ... persistent kernel" (one output tile per program,
// fp32 accumulator reset per tile, masked loads that read zero outside M/N/K,
// masked store) and the merged loop of "(3/n) ... cross tile pipelining".  How
// it is computed is this file's own design for MI355X:
//
//  * A workgroup owns a BM x BN output tile and walks K in BK slices.  Slices of
//    A (BM x BK) and B (BK x BN) are staged in LDS in a two-slot ring: while the
//    MFMAs consume slot s, the next slice travels from global memory into
//    registers and is written into slot s^1 before the single barrier of the
//    step.
//  * Both operands sit in LDS "K-contiguous": A as [m][k] (its natural layout),
//    B transposed to [n][k] on the way in (each loader thread reads an 8x8 or 4x8
//    (k x n) block with 16-byte row loads and transposes it in registers with
//    byte permutes), so that every MFMA operand fragment is one 16-byte LDS read.
//    The 16-byte chunks of each LDS row are XOR-swizzled by the row index (A:
//    row mod 8; B: (row mod 8) ^ (row/8 mod 4)) so that the 8 lanes served
//    together by the LDS touch 8 different bank groups on the fragment reads,
//    the A writes and (up to a factor of two) the B writes.  The swizzle term of
//    a fragment read depends only on the lane, so each lane keeps one LDS offset
//    per K sub-step and every read is that offset plus an immediate.
//  * The product uses v_mfma_f32_32x32x16_{f16,bf16}.  The operands are fed as
//    (B fragment, A fragment), so each 32x32 accumulator block holds C^T: a lane
//    owns 4 consecutive columns of one row, and the epilogue writes 8- or
//    16-byte vectors.
//  * Waves are arranged WM x WN over the tile; wave (wm, wn) owns a (BM/WM) x
//    (BN/WN) sub-tile of FM x FN accumulator blocks.  Fragments of K sub-step
//    s+1 are read from LDS while the MFMAs of sub-step s run; the last few MFMAs
//    of a K step are issued after the barrier, behind the first LDS reads of the
//    next slot.
//  * Global loads use a wave-uniform base pointer per row group plus one 32-bit
//    per-lane offset (the address arithmetic is scalar).
//  * Tile order and the persistent / flattened loops come from schedule.hpp; the
//    trace kernel runs the same functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "schedule.hpp"

namespace ts {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

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
    long long lda, ldb, ldc;  // strides between the stored rows, in elements: A [M][K] (lda = stride_am)
                              // or, on PATH_FULL_AT(BT), A stored [K][M] (lda = stride_ak); B [K][N]
                              // (ldb = stride_bk) or, on PATH_FULL_(AT)BT, B stored [N][K] (ldb =
                              // stride_bn); C [M][N]
    long long sam, sak, sbk, sbn;  // all four element strides (the masked path gathers with them)
    // Row alignment of A, B (16-bit elements) and C: 2 if rows allow 16-byte (A, B) /
    // full 4-element (C) vectors, 1 if they allow 4-byte (A, B) / 2-element (C) pieces,
    // 0 if only single elements.
    int vec_a, vec_b, vec_c;
    int c_align;              // largest of 16, 8, 4, 2 bytes dividing C's base and row pitch
    long long a_bytes, b_bytes;  // bytes from A (B) to the end of its last element
    SchedArgs s;
    unsigned long long* clk;  // null, or 4 values per program (see ProgramClock)
    // stream-K workspace (MODE_STREAMK launches that split tiles; see StreamK)
    float* sk_part;           // one partial tile (BM x BN fp32) per range
    int* sk_flags;            // one flag per range: 1 = its partial tile is written
    int* sk_err;              // incremented when a wait for a flag gives up
    int sk_spin;              // sleeps before a wait gives up
};

// Optional per-program clock record: shader-clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) at the program's start and end, written
// by thread 0 as clk[4p .. 4p+3] = {shader start, shader end, real start, real end}.
// The ratio of the two differences is the shader clock the program ran at.
struct ProgramClock {
    unsigned long long c0 = 0, r0 = 0;
    __device__ __forceinline__ void start(const GemmArgs& g) {
        if (g.clk) {
            c0 = __builtin_amdgcn_s_memtime();
            r0 = __builtin_amdgcn_s_memrealtime();
        }
    }
    __device__ __forceinline__ void stop(const GemmArgs& g) {
        if (g.clk) {
            const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
            if (threadIdx.x == 0) {
                unsigned long long* d = g.clk + 4 * (unsigned long long)blockIdx.x;
                d[0] = c0;
                d[1] = c1;
                d[2] = r0;
                d[3] = r1;
            }
        }
    }
};

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;             // threads
    static constexpr int TM = BM / WM, TN = BN / WN;    // wave sub-tile
    static constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 blocks per wave
    static constexpr int SUB = BK / 16;                 // MFMA K sub-steps per slice
    static constexpr int KCH = BK / 8;                  // 16-byte chunks per LDS row
    static constexpr int NA = BM * KCH;                 // A chunks per slice
    static constexpr int CA = (NA + NT - 1) / NT;       // A chunks per thread
    static constexpr int KBH = (BK * BN / 64 >= NT) ? 8 : 4;  // k rows of a B loader block
    static constexpr int NB = (BK / KBH) * (BN / 8);    // B loader blocks per slice
    static constexpr int CB = (NB + NT - 1) / NT;       // B blocks per thread
    static constexpr int ROW_BYTES = BK * 2;            // one LDS row (m or n) of a slice
    static constexpr int A_SLOT = BM * ROW_BYTES, B_SLOT = BN * ROW_BYTES;
    // LDS: A slots A0, A1, B slots B0, B1 and (BK = 64 tiles) a 4 KiB epilogue
    // staging area per wave, each its own array
    static constexpr int A_BYTES = 2 * A_SLOT, B_BYTES = 2 * B_SLOT;
    static constexpr int STAGE_W = 4096;
    static constexpr int C_BYTES = BK == 64 ? (NT / 64) * STAGE_W : 0;
    static constexpr int LDS_BYTES = A_BYTES + B_BYTES + C_BYTES;
    static constexpr int HOLD = (FM * FN >= 16) ? 8 : FM * FN / 2;  // MFMAs issued after the barrier
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave sub-tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0 && KCH <= 8 && (KCH & (KCH - 1)) == 0, "BK must be 16, 32 or 64");
    static_assert(BK % KBH == 0 && NT % KCH == 0, "loader shape");
    static_assert(A_SLOT <= 65535 && SUB % 2 == 0 || SUB == 1, "slot offsets must fit LDS immediates");
};

// ---- small device helpers ------------------------------------------------------

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

__device__ __forceinline__ uint32_t pack_bits(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// Output element conversion (round to nearest even) and stores of 4 consecutive
// columns; `vec` = all 4 inside N at an aligned address.
template <class TO> struct Out;
template <> struct Out<OutF32> {
    typedef float T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, int vec) {
        if (vec >= 2 && valid >= 4) {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        } else if (vec == 1 && valid >= 4) {
            reinterpret_cast<float2*>(p)[0] = make_float2(v[0], v[1]);
            reinterpret_cast<float2*>(p)[1] = make_float2(v[2], v[3]);
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = v[e];
        }
    }
};
template <> struct Out<OutF16> {
    typedef _Float16 T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, int vec) {
        _Float16 h[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        if (vec >= 1 && valid >= 4) {
            u32x2 w;
            w[0] = pack_bits(__builtin_bit_cast(uint16_t, h[0]), __builtin_bit_cast(uint16_t, h[1]));
            w[1] = pack_bits(__builtin_bit_cast(uint16_t, h[2]), __builtin_bit_cast(uint16_t, h[3]));
            if (vec >= 2) {
                *reinterpret_cast<u32x2*>(p) = w;
            } else {
                reinterpret_cast<uint32_t*>(p)[0] = w[0];
                reinterpret_cast<uint32_t*>(p)[1] = w[1];
            }
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = h[e];
        }
    }
};
template <> struct Out<OutBF16> {
    typedef __bf16 T;
    static __device__ __forceinline__ void store4(T* p, const float* v, int valid, int vec) {
        __bf16 h[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        if (vec >= 1 && valid >= 4) {
            u32x2 w;
            w[0] = pack_bits(__builtin_bit_cast(uint16_t, h[0]), __builtin_bit_cast(uint16_t, h[1]));
            w[1] = pack_bits(__builtin_bit_cast(uint16_t, h[2]), __builtin_bit_cast(uint16_t, h[3]));
            if (vec >= 2) {
                *reinterpret_cast<u32x2*>(p) = w;
            } else {
                reinterpret_cast<uint32_t*>(p)[0] = w[0];
                reinterpret_cast<uint32_t*>(p)[1] = w[1];
            }
        } else {
            for (int e = 0; e < 4; ++e) if (e < valid) p[e] = h[e];
        }
    }
};

// 16-bit elements p[0], p[stride], ..., p[7 stride], those at or past `valid` read
// as zero, packed as 8 consecutive values (a strided operand on the masked path).
__device__ __forceinline__ u32x4 gather8_masked(const uint16_t* p, long long stride, int valid) {
    uint32_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = (q < valid) ? (uint32_t)p[q * stride] : 0u;
    return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// 8 consecutive 16-bit elements p[0..7], those at or past `valid` read as zero.
// `vec` is the alignment level of p (2: 16 bytes, 1: 4 bytes, 0: 2 bytes).
__device__ __forceinline__ u32x4 load8_masked(const uint16_t* p, int valid, int vec) {
    if (valid >= 8) {
        if (vec >= 2) return *reinterpret_cast<const u32x4*>(p);
        if (vec == 1) {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
            return u32x4{q[0], q[1], q[2], q[3]};
        }
    }
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

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ u32x4 lds_read16(const char* lds, uint32_t off) {
    return *reinterpret_cast<const u32x4*>(lds + off);
}

// LDS transpose read (ds_read_b64_tr_b16).  Each lane addresses 4 consecutive
// 16-bit elements; within every group of 16 lanes, lane 4a + c receives element
// c of the chunks addressed by lanes a, a + 4, a + 8 and a + 12.
__device__ __forceinline__ u32x2 lds_read_tr(const char* lds, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) i16x4*)(lds + off)));
}

// ---- the tile engine -------------------------------------------------------------

// Two pipelines feed the MFMAs of a K step (64 MFMAs per wave for the big tiles):
//
//  fast (BK = 64, 128- or 256-wide tiles; whole tiles, or ragged edges that the
//    loads zero-fill themselves, see rsrc_a).  Both operands go straight
//    from global memory into LDS with direct-to-LDS buffer loads, no registers
//    in between:
//      A ([m][k], 16-byte chunks swizzled by swz(r) below) into two slots;
//      B in the slice's natural [k][n] layout (chunks swizzled by f(k) below)
//        into two slots, read back as MFMA operands with LDS transpose reads.
//    MFMA operand fragments are read two sub-steps (of 16 k) ahead into four
//    register buffers, so the workgroup barrier sits in the middle of a K step:
//    before it the MFMAs of sub-steps 0-1 run while the fragments of 2-3 are
//    read; the barrier certifies that every wave is done reading this slice and
//    that the next one has landed; after it the MFMAs of 2-3 run while the next
//    slice's first fragments are read and the slots this slice freed receive the
//    slices two ahead -- a full K step for every load to land.  The barrier
//    waits for every load of the step before (and nothing issued later).  Each
//    slot is its own LDS array and every slot index is a compile-time constant,
//    so the compiler can tell that a load into one slot never touches the slot
//    being read, and in the tiled and persistent loops the waits it places for
//    its own bookkeeping are already met by the explicit one (in the flattened
//    loop it still places a few full waits).  The cross-wave wait the pipeline
//    needs is explicit before the barrier.
//    The epilogue stages each wave's tile through a private 4 KiB of LDS, so that
//    every global store writes whole 128- or 256-byte row segments.  2 x 32 KiB
//    of A, 2 x 32 KiB of B and 8 x 4 KiB of staging fill the 160 KiB of LDS of
//    the 256 x 256 x 64 tile.
//  register (other masked shapes, or BK = 32): A and B one slice ahead in registers,
//    written at the last sub-steps into the other slot of two; B is transposed to
//    [n][k] with byte permutes on the way in.
// Kernel paths: whole tiles; masked register pipeline (any operand layout); direct-
// to-LDS pipeline with ragged edges zero-filled by the loads' range checks; whole
// tiles with B stored [N][K] (K contiguous, as A), whose B slices are staged and read
// exactly as A's; whole tiles with A stored [K][M] (M contiguous, as B), whose A
// slices are staged and read exactly as B's (with B stored [K][N] or [N][K]).
enum : int { PATH_FULL = 0, PATH_MASKED = 1, PATH_EDGE = 2, PATH_FULL_BT = 3, PATH_FULL_AT = 4, PATH_FULL_ATBT = 5 };

template <class Cfg, class TI, class TO, int PATH>
struct Engine {
    static constexpr bool MASKED = PATH == PATH_MASKED;
    static constexpr bool EDGE = PATH == PATH_EDGE;
    static constexpr bool BT = PATH == PATH_FULL_BT || PATH == PATH_FULL_ATBT;   // B stored [N][K]
    static constexpr bool AT = PATH == PATH_FULL_AT || PATH == PATH_FULL_ATBT;   // A stored [K][M]
    static constexpr bool EDGES = PATH != PATH_FULL;   // C stores masked to M x N
    static constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
    static constexpr int FM = Cfg::FM, FN = Cfg::FN, KCH = Cfg::KCH, SUB = Cfg::SUB;
    static constexpr int CA = Cfg::CA, CB = Cfg::CB, KBH = Cfg::KBH;
    static constexpr int RB = Cfg::ROW_BYTES;
    static constexpr int NW = NT / 64;               // waves
    static constexpr int NMF = FM * FN;              // MFMAs per sub-step
    static constexpr int A_ROWS_PER_C = NT / KCH;    // A rows between a thread's chunks
    static constexpr int NBN = BN / 8;               // B loader blocks along n
    static constexpr int RBB = BN * 2;               // bytes of one [k][n] B row (fast path)
    static constexpr int LPR = RBB / 16, RPD = 64 / LPR;   // B load lanes per row, rows per 1 KiB load
    static constexpr bool FAST_OK = RB == 128 && Cfg::C_BYTES > 0 && (BM * RB) % (1024 * NW) == 0 &&
                                    LPR >= 16 && LPR <= 64 && (LPR & (LPR - 1)) == 0 &&
                                    (BK * RBB) % (1024 * NW) == 0 && (NW * RPD) % 8 == 0 &&
                                    (BK * (RBB / 256)) % NW == 0;
    static constexpr bool FAST = !MASKED && FAST_OK;
    static_assert(!EDGE || FAST, "the edge paths run the direct-to-LDS pipeline");
    static constexpr int BH = RBB / 256;                                // 256-byte pieces of a B row
    static constexpr int A_DMA_N = FAST ? BM * RB / 1024 / NW : 0;   // 1 KiB A loads per wave
    static constexpr int B_DMA_N = !FAST ? 0 : BT ? BN * RB / 1024 / NW   // 1 KiB B loads per wave
                                                  : BK * RBB / 1024 / NW;
    static_assert(!BT || FAST, "B stored [N][K] runs on the direct-to-LDS pipeline");
    // A stored [K][M]: its [k][m] slices have the geometry of B's [k][n] slices
    static_assert(!AT || (FAST && BM == BN), "A stored [K][M] runs on the direct-to-LDS pipeline of square tiles");
    static constexpr int DA = FAST ? 2 : 1;          // A slices in flight ahead of the multiplied one
    static constexpr int DB = FAST ? 2 : 1;          // B slices in flight ahead of the multiplied one
    static constexpr int NFB = FAST ? 4 : 2;         // fragment register buffers
    static constexpr int NJB = FN < 4 ? FN : 4;      // per-lane B transpose-read offsets
    static constexpr int NIA = FM < 4 ? FM : 4;      // per-lane A transpose-read offsets (A stored [K][M])
    // sub-steps that write the next slice into LDS (register path)
    static constexpr int A_STORE_S = SUB > 2 ? SUB - 2 : SUB - 1;
    static constexpr int B_STORE_S = SUB - 1;
    static_assert(CB == 1, "one B loader block per thread");

    const GemmArgs& g;
    char* la[2];          // A slots
    char* lb[2];          // B slots
    char* ldsc;           // epilogue staging (fast path)
    int tid, lane, wm, wn, wave;

    // per-lane LDS byte offsets
    uint32_t a_rd[SUB];   // A fragment read of block 0 at sub-step s (block i: + i*32*RB)
    uint32_t b_rd[SUB];   // register path: B fragment read, as a_rd
    uint32_t bt_rd[NJB];  // fast path: B transpose read of block u (block j: bt_rd[j % 4] + (j / 4) * 256)
    uint32_t b_dg[2];     // fast path: B load global offset, by bit 3 of its first row
    uint32_t at_rd[NIA];  // A stored [K][M]: A transpose read of block u, as bt_rd
    uint32_t a_dg[2];     // A stored [K][M]: A load global offset, as b_dg
    uint32_t a_wr[2];     // register path: A chunk c at a_wr[c&1] + c*A_ROWS_PER_C*RB
    uint32_t b_wr[8];     // B write j of the loader block (see b_wr_at)
    uint32_t b_sel[2];    // register path: byte-permute selector of B writes with even / odd j
    // per-lane global byte offsets
    uint32_t a_go[2], b_go;   // A: [c&1] of the load / chunk index c
    uint32_t bt_go[2];        // PATH_FULL_BT: B's load offsets, as a_go
    uint32_t a_kc[2];         // edge paths: first k (element) of the A chunk a_go[e] points at
    int klim = 0;             // edge paths: k elements of the A slice being loaded that exist
    bool b_active;        // this thread owns a B loader block

    u32x4 ra[FAST ? 1 : CA];                 // A slice in flight (register path)
    u32x4 rb[1][KBH];                        // B slice in flight (register path; KBH rows of 8 columns)
    u32x4 fa[NFB][FM], fb[NFB][FN];
    f32x16 acc[FM][FN];

    __device__ __forceinline__ Engine(const GemmArgs& g_, char* a0, char* a1, char* b0, char* b1, char* lds_c)
        : g(g_), la{a0, a1}, lb{b0, b1}, ldsc(lds_c) {
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        wm = wave / Cfg::WN;
        wn = wave % Cfg::WN;
        const int r32 = lane & 31, hk = lane >> 5;
        // Rows of [m][k] (and, on the register path, [n][k]) slices are swizzled by
        // swz(r) = (r ^ (r >> 3)) mod KCH.  A fragment row is (32-aligned base) +
        // r32, so swz depends on r32 and, for KCH = 8, on bit 0 of the block index
        // (bit 5 of the row), which flips chunk bit 2, i.e. sub-step s <-> s ^ 2:
        // odd blocks use the offset of s ^ 2.
        const int sw = (r32 ^ (r32 >> 3)) & (KCH - 1);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const int ch = 2 * s + hk;
            a_rd[s] = (uint32_t)((wm * Cfg::TM + r32) * RB + ((ch ^ sw) * 16));
            b_rd[s] = (uint32_t)((wn * Cfg::TN + r32) * RB + ((ch ^ sw) * 16));
        }
        const int nb = tid % NBN, kb = tid / NBN;   // B loader block (kb, nb) of this thread
        b_active = Cfg::NB % NT == 0 || tid < Cfg::NB;
        b_go = (uint32_t)(((long long)kb * KBH * g.ldb + nb * 8) * 2);
        if (FAST) {
            // A: lane l of a 1 KiB load lands at row (8 * grp + l/8), chunk l%8 of
            // the slot and fetches the logical chunk the swizzle puts there; with
            // grp = c * NW + wave, grp mod 8 depends on c only through bit 2 of
            // c * NW (4 waves: even and odd c differ; 8 waves: never)
            const int row = lane >> 3, pc = lane & 7;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int grp7 = (4 * e + wave) & 7;
                a_go[e] = (uint32_t)(((long long)row * g.lda + ((pc ^ row ^ grp7) * 8)) * 2);
                a_kc[e] = (uint32_t)((pc ^ row ^ grp7) * 8);
                a_wr[e] = 0;
                // B stored [N][K]: its [n][k] slot is filled exactly as A's [m][k] slot
                bt_go[e] = (uint32_t)(((long long)row * g.ldb + ((pc ^ row ^ grp7) * 8)) * 2);
            }
            // B: [k][n] rows whose 16-byte chunks are XOR-swizzled by
            //   f(k) = 4 (k mod 4) ^ 2 (bit 3 of k),
            // so that the 4 k rows x 64 bytes that 32 lanes of a transpose read
            // touch (and the 8 rows x 32 bytes of lanes 0-15 with 32-47) fall in
            // distinct banks.  Transpose read: lane j of 16-lane group q addresses
            // row 16 s + 8 hk + 4 rd + j/4 (hk = q/2), columns 16 (q mod 2) +
            // 4 (j mod 4) of its 32-column block, so that lane 16 q + i ends up with
            // 4 consecutive k of column i + 16 (q mod 2); two reads (rd = 0, 1) make
            // the 8 k values of its MFMA operand.  There k mod 4 = j/4 and bit 3 of
            // k = hk, so the swizzle is fixed per lane.
            const int q = lane >> 4, j = lane & 15;
            const int qh = q >> 1, qn = q & 1, e = j >> 2, a = j & 3;
            const int ff = (4 * e) ^ (2 * qh);
#pragma unroll
            for (int u = 0; u < NJB; ++u) {
                const int W = wn * FN + u;   // 32-column block within the tile
                const int chunk = ((4 * W) | (2 * qn + (a >> 1))) ^ ff;
                bt_rd[u] = (uint32_t)((8 * qh + e) * RBB + chunk * 16 + (a & 1) * 8);
            }
            // B loads: lane l lands at row RPD * grp + l / LPR, chunk l mod LPR, and
            // fetches the logical chunk the swizzle puts there; bit 3 of the row
            // varies with the load index c through c * NW * RPD (a multiple of 8)
            const int rl = lane / LPR, pch = lane % LPR;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int r = 8 * e2 + wave * RPD + rl;
                const int fr = (4 * (r & 3)) ^ (2 * ((r >> 3) & 1));
                b_dg[e2] = (uint32_t)(((long long)rl * g.ldb + (pch ^ fr) * 8) * 2);
                a_dg[e2] = (uint32_t)(((long long)rl * g.lda + (pch ^ fr) * 8) * 2);
            }
            // A stored [K][M]: its [k][m] slot is filled and read exactly as B's [k][n]
            // slot, with 32-row blocks of m in place of 32-column blocks of n
#pragma unroll
            for (int u = 0; u < NIA; ++u) {
                const int W = wm * FM + u;   // 32-row block within the tile
                const int chunk = ((4 * W) | (2 * qn + (a >> 1))) ^ ff;
                at_rd[u] = (uint32_t)((8 * qh + e) * RBB + chunk * 16 + (a & 1) * 8);
            }
            b_wr[0] = 0;
            b_sel[0] = b_sel[1] = 0;
        } else {
            // A chunk (row, kc) of this thread; chunk c adds c * A_ROWS_PER_C rows,
            // which changes the swizzle only through bit 2 for odd c (KCH = 8)
            const int row = tid / KCH, kc = tid % KCH;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = row + e * A_ROWS_PER_C;
                a_wr[e] = (uint32_t)(r * RB + ((kc ^ ((r ^ (r >> 3)) & (KCH - 1))) * 16)) - e * A_ROWS_PER_C * RB;
                a_go[e] = (uint32_t)(((long long)row * g.lda + kc * 8) * 2);
            }
            // B is transposed to [n][k]: write instruction j of lane group half
            // h = (nb >> 3) & 1 stores column j ^ h, so that the 16 lanes served
            // together cover both row parities and 16 distinct bank groups.  Its
            // LDS row is n = 8 nb + (j ^ h) and its chunk (c0 ^ swz(n)) with
            // swz(n) = (j ^ h ^ nb) mod 8; with 128-byte rows the offset is
            //   base + ((j ^ h) * 128) + ((x ^ j) * 16),  x = (c0 ^ h ^ nb) mod 8,
            // whose variable bits 4..9 sit above and apart from base's, so it equals
            // b_wr ^ (j * 144) with b_wr = base | (h * 128) | (x * 16).
            const int h = (nb >> 3) & 1;
            b_sel[0] = h ? 0x07060302u : 0x05040100u;   // even j: half (j ^ h) & 1
            b_sel[1] = h ? 0x05040100u : 0x07060302u;   // odd j
            if (KCH == 8) {
                const int c0 = KBH == 8 ? kb : (kb >> 1);
                const int x = (c0 ^ h ^ nb) & 7;
                const uint32_t base = (uint32_t)(nb * 8 * RB + (KBH == 8 ? 0 : (kb & 1) * 8));
                b_wr[0] = base | (uint32_t)(h * 128) | (uint32_t)(x * 16);
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int n = nb * 8 + (jj ^ h);
                    const int swz = (n ^ (n >> 3)) & (KCH - 1);
                    if (KBH == 8)
                        b_wr[jj] = (uint32_t)(n * RB + ((kb ^ swz) * 16));
                    else
                        b_wr[jj] = (uint32_t)(n * RB + ((((kb >> 1) ^ swz)) * 16) + (kb & 1) * 8);
                }
            }
        }
        // Keep the lane offsets opaque: otherwise their compile-time parts (the B
        // region starts at 64 KiB or more) are folded into per-access constants too
        // large for the 16-bit LDS offset field, and every access needs its own
        // register.
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            if (!AT) asm volatile("" : "+v"(a_rd[s]));
            if (!FAST || BT) asm volatile("" : "+v"(b_rd[s]));
        }
        if (AT) {
#pragma unroll
            for (int u = 0; u < NIA; ++u) asm volatile("" : "+v"(at_rd[u]));
        }
        if (FAST && !BT) {
#pragma unroll
            for (int u = 0; u < NJB; ++u) asm volatile("" : "+v"(bt_rd[u]));
        } else {
            asm volatile("" : "+v"(a_wr[0]));
            asm volatile("" : "+v"(a_wr[1]));
        }
        if (FAST) {
        } else if (KCH == 8) {
            asm volatile("" : "+v"(b_wr[0]));
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) asm volatile("" : "+v"(b_wr[jj]));
        }
    }

    __device__ __forceinline__ void zero_acc() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    // Scalar-register buffer resource over `p` with `nrec` records: -1 (all) for a
    // slice that exists, 0 past the last one, which turns every load through it
    // into a zero with no memory access.  The count is an integer computed with
    // scalar arithmetic (see vmask): a select on a bool is materialised in a vector
    // register, which drags the whole resource into vector registers and makes the
    // compiler wrap every load in a loop over distinct lane values.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t* p, int nrec) const {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0,
                                                 __builtin_amdgcn_readfirstlane(nrec), kBufferFlags);
    }
    // -1 if k < lim, else 0 (for 0 <= k, lim < 2^30).  RFL: k and lim are
    // wave-uniform but the compiler's divergence analysis cannot see it (in the
    // stream-K kernel, whose fix-up wait is a branch taken by one lane), so the
    // difference goes through readfirstlane.
    template <bool RFL = false>
    static __device__ __forceinline__ int vmask(int k, int lim) {
        int d = RFL ? __builtin_amdgcn_readfirstlane(k - lim) : k - lim;
        asm("" : "+s"(d));  // opaque: keeps the shift from being folded back into a compare and select
        return d >> 31;
    }

    // Fast path: one direct-to-LDS load of 16 bytes per lane; lane l's bytes land at
    // dst + 16 l.
    static __device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& r, uint32_t voff, int soff, char* dst) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff, soff, 0, 0);
    }

    // Buffer resource over the slice at element offset `off` of A (B): on the edge
    // path its record count stops at the matrix's last element, so that rows past
    // M (K) and columns past the end read as zero.  Every offset of those loads is
    // in the per-lane offset, which the range check covers; the check is made per
    // dword, so each dword of a load reads either its data or zero (A: K, lda and
    // the base are multiples of 8 elements, so a chunk never mixes the last k of a
    // row with the next row; B: N, ldb and the base are even / 4-byte aligned, so
    // no dword straddles the end of B).
    // The count is clamped to [0, 2^31 - 16], a multiple of 4; the in-tile offsets
    // of the edge path stay below 2^30.
    static __device__ __forceinline__ int clamp_records(long long left) {
        return (int)(left < 0 ? 0 : left < 0x7ffffff0LL ? left : 0x7ffffff0LL);
    }
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_a(long long off, int valid) const {
        if constexpr (!EDGE) return rsrc(g.A + off, valid);
        return rsrc(g.A + off, clamp_records(g.a_bytes - 2 * off) & valid);
    }
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(long long off, int valid) const {
        if constexpr (!EDGE) return rsrc(g.B + off, valid);
        return rsrc(g.B + off, clamp_records(g.b_bytes - 2 * off) & valid);
    }
    // A per-lane offset no record count reaches: the load reads zero.
    static constexpr uint32_t kOutOfRange = 0x80000000u;

    // Fast path: 1 KiB A load number c of this wave, into A slot `slot`.  Edge
    // paths: chunks at or past k = klim of the slice read as zero.
    template <int SLOT>
    __device__ __forceinline__ void dma_a_one(int c, const __amdgpu_buffer_rsrc_t& r) {
        if constexpr (AT) {   // as B's [k][n] loads, over A's [k][m] rows
            const int grp = c * NW + wave;
            const int e = ((c * NW * RPD) >> 3) & 1;
            dma16(r, a_dg[e], (int)((long long)grp * RPD * g.lda * 2), la[SLOT] + grp * 1024);
            return;
        }
        const int grp = c * NW + wave;                     // 8-row group (1 KiB)
        const int e = ((c * NW) >> 2) & 1;
        if constexpr (EDGE) {
            const uint32_t voff = a_go[e] + (uint32_t)(grp * 8 * (int)g.lda * 2);
            dma16(r, (int)a_kc[e] < klim ? voff : kOutOfRange, 0, la[SLOT] + grp * 1024);
        } else {
            dma16(r, a_go[e], (int)((long long)grp * 8 * g.lda * 2), la[SLOT] + grp * 1024);
        }
    }
    // Element offset of A's slice k of tile row m0 (the slice's first element).
    __device__ __forceinline__ long long a_slice(int m0, int k) const {
        return AT ? (long long)k * BK * g.lda + m0 : (long long)m0 * g.lda + k * BK;
    }
    template <int SLOT>
    __device__ __forceinline__ void dma_a(int m0, int k, int valid) {
        const __amdgpu_buffer_rsrc_t r = rsrc_a(a_slice(m0, k), valid);
        if constexpr (EDGE) klim = g.K - k * BK;
#pragma unroll
        for (int c = 0; c < A_DMA_N; ++c) dma_a_one<SLOT>(c, r);
    }
    // Fast path: B load number c of this wave (1 KiB, 16 bytes a lane), into B slot
    // `slot`.  On the edge path B's rows need only be 4-byte aligned: a 16-byte
    // buffer load needs no more than dword alignment, and the range check of a raw
    // buffer load is made per dword (both checked on MI355X with an in-bounds probe),
    // so a load that straddles the end of B returns its dwords before the end and
    // zeros after it.
    // Element offset of B's slice k of tile column n0 (the slice's first element).
    __device__ __forceinline__ long long b_slice(int n0, int k) const {
        return BT ? (long long)n0 * g.ldb + k * BK : (long long)k * BK * g.ldb + n0;
    }
    template <int SLOT>
    __device__ __forceinline__ void dma_b_one(int c, const __amdgpu_buffer_rsrc_t& r) {
        if constexpr (BT) {   // as dma_a_one, over B's [n][k] rows
            const int grp = c * NW + wave;
            const int e = ((c * NW) >> 2) & 1;
            dma16(r, bt_go[e], (int)((long long)grp * 8 * g.ldb * 2), lb[SLOT] + grp * 1024);
            return;
        }
        const int grp = c * NW + wave;                 // RPD-row group (1 KiB)
        const int e = ((c * NW * RPD) >> 3) & 1;
        if constexpr (EDGE)
            dma16(r, b_dg[e] + (uint32_t)(grp * RPD * (int)g.ldb * 2), 0, lb[SLOT] + grp * 1024);
        else
            dma16(r, b_dg[e], (int)((long long)grp * RPD * g.ldb * 2), lb[SLOT] + grp * 1024);
    }
    template <int SLOT>
    __device__ __forceinline__ void dma_b(int n0, int k, int valid) {
        const __amdgpu_buffer_rsrc_t r = rsrc_b(b_slice(n0, k), valid);
#pragma unroll
        for (int c = 0; c < B_DMA_N; ++c) dma_b_one<SLOT>(c, r);
    }

    // A slice k of tile row m0 into registers (register path).
    __device__ __forceinline__ void load_a(int m0, int k, int valid) {
        const int k0 = k * BK;
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t r = rsrc(g.A + (long long)m0 * g.lda + k0, valid);
#pragma unroll
            for (int c = 0; c < CA; ++c) {
                const int soff = (int)(c * A_ROWS_PER_C * g.lda * 2);
                ra[c] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)a_go[0], soff, 0);
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            const int idx = c * NT + tid;
            const int row = idx / KCH, kc = idx % KCH;
            const int gm = m0 + row, gk = k0 + kc * 8;
            const bool in = valid && (Cfg::NA % NT == 0 || idx < Cfg::NA) && gm < g.M;
            if (!in)
                ra[c] = u32x4{0, 0, 0, 0};
            else if (g.sak == 1)
                ra[c] = load8_masked(g.A + (long long)gm * g.lda + gk, g.K - gk, g.vec_a);
            else   // A stored [K][M]: 8 consecutive k of row gm, g.sak apart
                ra[c] = gather8_masked(g.A + (long long)gm * g.sam + (long long)gk * g.sak, g.sak, g.K - gk);
        }
    }

    // B row q of slice k, tile column n0, into register set SET (unmasked).
    template <int SET>
    __device__ __forceinline__ void load_b_row(int q, const __amdgpu_buffer_rsrc_t& r) {
        const int soff = (int)(q * g.ldb * 2);
        // threads without a B block re-read thread 0's block (in bounds); the value
        // is never stored
        rb[SET][q] = __builtin_amdgcn_raw_buffer_load_b128(r, (Cfg::NB % NT == 0 || b_active) ? (int)b_go : 0, soff, 0);
    }

    // B slice k of tile column n0 into register set SET.
    template <int SET>
    __device__ __forceinline__ void load_b(int n0, int k, int valid) {
        const int k0 = k * BK;
        if (!MASKED) {
            const __amdgpu_buffer_rsrc_t r = rsrc(g.B + (long long)k0 * g.ldb + n0, valid);
#pragma unroll
            for (int q = 0; q < KBH; ++q) load_b_row<SET>(q, r);
            return;
        }
        const int nb = tid % NBN, kb = tid / NBN;
        const int gn = n0 + nb * 8, gk = k0 + kb * KBH;
#pragma unroll
        for (int q = 0; q < KBH; ++q) {
            if (!(valid && b_active && gk + q < g.K))
                rb[SET][q] = u32x4{0, 0, 0, 0};
            else if (g.sbn == 1)
                rb[SET][q] = load8_masked(g.B + (long long)(gk + q) * g.ldb + gn, g.N - gn, g.vec_b);
            else   // B stored [N][K]: 8 consecutive n of row gk + q, g.sbn apart
                rb[SET][q] = gather8_masked(g.B + (long long)(gk + q) * g.sbk + (long long)gn * g.sbn, g.sbn,
                                            g.N - gn);
        }
    }

    // Register A slice -> LDS slot SLOT (register path).
    template <int SLOT>
    __device__ __forceinline__ void store_a() {
        char* sa = la[SLOT];
#pragma unroll
        for (int c = 0; c < CA; ++c) {
            if (Cfg::NA % NT == 0 || c * NT + tid < Cfg::NA)
                *reinterpret_cast<u32x4*>(sa + a_wr[c & 1] + c * A_ROWS_PER_C * RB) = ra[c];
        }
    }

    // Number of LDS writes of one B slice per thread (register path).
    static constexpr int NBW = FAST ? 0 : 8;

    // LDS offset of B write j (slot 0).
    __device__ __forceinline__ uint32_t b_wr_at(int j) const {
        return KCH == 8 ? (b_wr[0] ^ (uint32_t)(j * 144)) : b_wr[j];
    }

    // Write j of register set SET into B slot SLOT (register path): column j ^ h
    // of the loader block (see b_wr), transposed.
    template <int SET, int SLOT>
    __device__ __forceinline__ void store_b_one(int j) {
        if (!(Cfg::NB % NT == 0) && !b_active) return;
        char* sb = lb[SLOT];
        const int d = j >> 1;
        const uint32_t sel = b_sel[j & 1];
        if (KBH == 8) {
            u32x4 col;
#pragma unroll
            for (int q = 0; q < 4; ++q) col[q] = __builtin_amdgcn_perm(rb[SET][2 * q + 1][d], rb[SET][2 * q][d], sel);
            *reinterpret_cast<u32x4*>(sb + b_wr_at(j)) = col;
        } else {
            u32x2 col;
#pragma unroll
            for (int q = 0; q < 2; ++q) col[q] = __builtin_amdgcn_perm(rb[SET][2 * q + 1][d], rb[SET][2 * q][d], sel);
            *reinterpret_cast<u32x2*>(sb + b_wr_at(j)) = col;
        }
    }

    template <int SET, int SLOT>
    __device__ __forceinline__ void store_b() {
#pragma unroll
        for (int j = 0; j < NBW; ++j) store_b_one<SET, SLOT>(j);
    }

    // A fragment of 32-row block i at sub-step s from slot SLOT.
    template <int SLOT>
    __device__ __forceinline__ u32x4 read_a(int s, int i) const {
        if constexpr (AT) {   // two transpose reads, as read_b's
            const char* tb = la[SLOT] + (i >> 2) * 256 + 16 * s * RBB;
            const u32x2 lo = lds_read_tr(tb, at_rd[i & 3]);
            const u32x2 hi = lds_read_tr(tb + 4 * RBB, at_rd[i & 3]);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        const char* base = la[SLOT];
        return lds_read16(base, a_rd[(KCH == 8 && (i & 1)) ? (s ^ 2) : s] + i * 32 * RB);
    }

    // B fragment of 32-column block j at sub-step s from slot SLOT.
    template <int SLOT>
    __device__ __forceinline__ u32x4 read_b(int s, int j) const {
        if (FAST && !BT) {   // two transpose reads: k offsets 0-3 and 4-7 of the lane's half
            const char* base = lb[SLOT] + (j >> 2) * 256 + 16 * s * RBB;
            const u32x2 lo = lds_read_tr(base, bt_rd[j & 3]);
            const u32x2 hi = lds_read_tr(base + 4 * RBB, bt_rd[j & 3]);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        return lds_read16(lb[SLOT], b_rd[(KCH == 8 && (j & 1)) ? (s ^ 2) : s] + j * 32 * RB);
    }

    template <int SLOT>
    __device__ __forceinline__ void read_frags(int s, int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = read_a<SLOT>(s, i);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = read_b<SLOT>(s, j);
    }

    // Fragment number idx of sub-step s, in the order the MFMAs of a sub-step
    // first need them: A block 0, the B blocks, then A blocks 1, 2, ...
    template <int SLOT>
    __device__ __forceinline__ void read_frag(int s, int idx, int buf) {
        if (idx == 0)
            fa[buf][0] = read_a<SLOT>(s, 0);
        else if (idx <= FN)
            fb[buf][idx - 1] = read_b<SLOT>(s, idx - 1);
        else
            fa[buf][idx - FN] = read_a<SLOT>(s, idx - FN);
    }

    // MFMA number t of a sub-step, in (i, j) order.
    __device__ __forceinline__ void mfma_one(int buf, int t) {
        const int i = t / FN, j = t % FN;
        acc[i][j] = mfma32<TI>(fb[buf][j], fa[buf][i], acc[i][j]);
    }

    // MFMAs number [first, last) of a sub-step, in (i, j) order.
    __device__ __forceinline__ void mfmas(int buf, int first, int last) {
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            if (t < first || t >= last) continue;
            const int i = t / FN, j = t % FN;
            acc[i][j] = mfma32<TI>(fb[buf][j], fa[buf][i], acc[i][j]);
        }
    }

    // Slices loaded by a K step: A slice ka of tile row origin m0 (DA slices ahead
    // of the one multiplied) and B slice kb of tile column origin n0 (DB ahead).
    // A zero `v*` means past the last slice: nothing is read and zeros flow.
    struct Next {
        int m0, ka;
        int va;    // record-count mask: -1 for a slice that exists, 0 past the last
        int n0, kb;
        int vb;
    };

    // Issue plan of the unmasked paths over the MFMA slots of a K step (global slot
    // index gt = S * NMF + t): the VMEM loads and the B writes into LDS are spread
    // over the whole step, one per few MFMAs, so that neither the texture path nor
    // the LDS ever backs up far enough to stall the wave's in-order issue while
    // the matrix unit waits; each slot also carries at most one fragment read for
    // the next sub-step.  Loads come first (B, then A), then the B writes.
    static constexpr int NBL = FAST ? B_DMA_N : KBH;           // B loads per step
    static constexpr int NVM = NBL + (FAST ? A_DMA_N : CA);   // VMEM loads per step
    static constexpr int NSLOT = SUB * NMF - Cfg::HOLD;       // MFMA slots before the barrier
    // Small tiles have too few MFMA slots: all loads at slot 0, all B writes after
    // the last sub-step's MFMAs.
    static constexpr bool SPREAD = NSLOT >= NVM + NBW;
    static constexpr int VM_STRIDE = NSLOT >= 3 * (NVM + NBW) ? 3 : (NSLOT >= 2 * (NVM + NBW) ? 2 : 1);
    static constexpr int VM_FIRST = 1;                                        // loads at VM_FIRST + i*VM_STRIDE
    static constexpr int ST_FIRST = SPREAD ? VM_FIRST + NVM * VM_STRIDE : 1 << 20;  // B writes at ST_FIRST + j*VM_STRIDE
    static_assert(NVM < 64, "vmcnt range");

    // Register path (unmasked): load number vi of a step.
    template <int BSET>
    __device__ __forceinline__ void issue_load(int vi, const __amdgpu_buffer_rsrc_t& ra_rsrc,
                                               const __amdgpu_buffer_rsrc_t& rb_rsrc) {
        if (vi < KBH) {
            load_b_row<BSET>(vi, rb_rsrc);
        } else {
            const int c = vi - KBH;
            const int soff = (int)(c * A_ROWS_PER_C * g.lda * 2);
            ra[c] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, (int)a_go[0], soff, 0);
        }
    }

    // Sub-step S of a K step on B slot SLOT.
    template <int SLOT, int S>
    __device__ __forceinline__ void substep(const Next& nx) {
        constexpr int b = S & 1;
        constexpr bool last = S + 1 == SUB;
        constexpr int nmf = last ? NMF - Cfg::HOLD : NMF;
        constexpr int NFR = last ? 0 : FM + FN;        // fragment reads to spread
        if (MASKED) {
            if (S == 0) {
                load_b<0>(nx.n0, nx.kb, nx.vb);
                load_a(nx.m0, nx.ka, nx.va);
            }
            if (!last) read_frags<SLOT>(S + 1, b ^ 1);
            if (S == A_STORE_S) store_a<SLOT ^ 1>();
            if (S == B_STORE_S) store_b<0, SLOT ^ 1>();
            mfmas(b, 0, nmf);
            __builtin_amdgcn_sched_barrier(0);
            return;
        }
        constexpr int NT_ = (nmf > NFR ? nmf : NFR);
        const __amdgpu_buffer_rsrc_t rb_rsrc = rsrc(g.B + (long long)nx.kb * BK * g.ldb + nx.n0, nx.vb);
        const __amdgpu_buffer_rsrc_t ra_rsrc = rsrc(g.A + (long long)nx.m0 * g.lda + nx.ka * BK, nx.va);
#pragma unroll
        for (int t = 0; t < NT_; ++t) {
            const int gt = S * NMF + t;
            if (t < nmf) mfma_one(b, t);
            if (t < NFR) read_frag<SLOT>(S + 1 < SUB ? S + 1 : 0, t, b ^ 1);
            if (SPREAD) {
                const int vi = (gt - VM_FIRST) / VM_STRIDE;  // load number at this slot
                if (gt >= VM_FIRST && (gt - VM_FIRST) % VM_STRIDE == 0 && vi < NVM)
                    issue_load<0>(vi, ra_rsrc, rb_rsrc);
            } else if (gt == 0) {
#pragma unroll
                for (int vi = 0; vi < NVM; ++vi) issue_load<0>(vi, ra_rsrc, rb_rsrc);
            }
            const int wi = (gt - ST_FIRST) / VM_STRIDE;  // B write number at this slot
            if (gt >= ST_FIRST && (gt - ST_FIRST) % VM_STRIDE == 0 && wi < NBW) store_b_one<0, SLOT ^ 1>(wi);
            if (S == A_STORE_S && t < CA) {
                if (Cfg::NA % NT == 0 || t * NT + tid < Cfg::NA)
                    *reinterpret_cast<u32x4*>(la[SLOT ^ 1] + a_wr[t & 1] + t * A_ROWS_PER_C * RB) = ra[t];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // B writes that did not fit before the barrier slots
        if (last) {
#pragma unroll
            for (int wj = 0; wj < NBW; ++wj)
                if (ST_FIRST + wj * VM_STRIDE >= S * NMF + NT_) store_b_one<0, SLOT ^ 1>(wj);
        }
    }

    template <int SLOT, int... S>
    __device__ __forceinline__ void substeps(const Next& nx, std::integer_sequence<int, S...>) {
        (substep<SLOT, S>(nx), ...);
    }

    // Fast path barrier: this wave's loads older than its last `pending` VMEM
    // operations (they return in order) have landed and its LDS accesses are
    // done; then the workgroup meets.
    template <int pending>
    __device__ __forceinline__ void barrier_after_loads() {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(pending) : "memory");
    }

    // One K step over B slot SLOT (fragments of its sub-step 0 already in buffer
    // 0).  Slot SLOT^1 (and on the fast path the A ring slot two ahead), which
    // every wave finished reading before the last barrier, receives a later slice;
    // after this step's barrier the sub-step 0 fragments of the next slot are
    // read, behind the last HOLD MFMAs of this step.  Past the last slice these
    // writes and reads carry zeros nobody uses, so every step has the same shape
    // and the accumulators stay in one set of registers through the loop.
    // Fast path, sub-step S of a K step on B slot SLOT: the MFMAs of sub-step S
    // (fragment buffer S) with the reads of the fragments of sub-step S + 2 mod 4
    // (into its buffer) spread over them -- of this slice for S < 2, of the next
    // one (slot SLOT^1) for S >= 2 -- and, for S >= 2, the loads into the slots
    // this slice freed: B (slice nx.kb), then A (slice nx.ka), into slot SLOT.
    static constexpr int F_NFR = FM + FN;                            // fragment reads per sub-step
    static constexpr int F_DS = 2 * NMF >= 2 * NVM ? 2 : 1;          // MFMA slots between loads
    static constexpr int F_PER = (NVM + 2 * NMF - 1) / (2 * NMF);    // loads per such slot
    template <int SLOT, int S>
    __device__ __forceinline__ void fast_sub(const __amdgpu_buffer_rsrc_t& ra_, const __amdgpu_buffer_rsrc_t& rb_) {
        constexpr int RS = (S + 2) & 3;
        constexpr int RSLOT = S < 2 ? SLOT : (SLOT ^ 1);
        constexpr int NT_ = NMF > F_NFR ? NMF : F_NFR;
#pragma unroll
        for (int t = 0; t < NT_; ++t) {
            if (t < NMF) mfma_one(S, t);
            if (t < F_NFR) read_frag<RSLOT>(RS, t, RS);
            if (S >= 2) {
                const int gt = (S - 2) * NMF + t;
                if (gt % F_DS == 0) {
#pragma unroll
                    for (int d = 0; d < F_PER; ++d) {
                        const int vi = (gt / F_DS) * F_PER + d;
                        if (vi < B_DMA_N)
                            dma_b_one<SLOT>(vi, rb_);
                        else if (vi < NVM)
                            dma_a_one<SLOT>(vi - B_DMA_N, ra_);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // `after_store`: the epilogue stores of the tile before were issued after the
    // loads this barrier waits for; those of store class `sc` (store_class) may
    // stay in flight.  The default counts the unmasked epilogue's stores, and none
    // on the edge path, whose masked epilogue issues a varying number.
    template <int SLOT>
    __device__ __forceinline__ void kstep(const Next& nx, bool after_store = false, int sc = EDGE ? 0 : 1) {
        if constexpr (FAST) {
            kstep_at<SLOT>(a_slice(nx.m0, nx.ka), b_slice(nx.n0, nx.kb), nx.ka, nx.va, after_store, sc);
            return;
        }
        constexpr int LB = (SUB - 1) & 1;  // fragment buffer of the last sub-step
        substeps<SLOT>(nx, std::make_integer_sequence<int, SUB>{});
        __syncthreads();
        read_frags<SLOT ^ 1>(0, 0);
        mfmas(LB, NMF - Cfg::HOLD, NMF);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Fast path: the K step above with the slices it loads given by their element
    // offsets in A and B (slice k within its tile, record-count mask v).
    // ENDS: the last K step of a tile whose epilogue follows, in a loop that reads
    // the next slice's first fragments again after the epilogue; its barrier then
    // only has to certify that every wave has finished reading this slot, and the
    // wait for the next slice moves behind the epilogue.
    template <int SLOT, bool ENDS = false>
    __device__ __forceinline__ void kstep_at(long long a_off, long long b_off, int k, int v, bool after_store,
                                             int sc) {
        static_assert(FAST, "direct-to-LDS pipeline");
        const __amdgpu_buffer_rsrc_t rb_ = rsrc_b(b_off, v);
        const __amdgpu_buffer_rsrc_t ra_ = rsrc_a(a_off, v);
        if constexpr (EDGE) klim = g.K - k * BK;
        fast_sub<SLOT, 0>(ra_, rb_);
        fast_sub<SLOT, 1>(ra_, rb_);
        if constexpr (ENDS)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if (after_store)
            barrier_behind_stores<0>(sc);
        else
            barrier_after_loads<0>();
        fast_sub<SLOT, 2>(ra_, rb_);
        fast_sub<SLOT, 3>(ra_, rb_);
    }
    // Element distance between consecutive slices of A (B).
    __device__ __forceinline__ long long a_kstride() const { return AT ? (long long)BK * g.lda : BK; }
    __device__ __forceinline__ long long b_kstride() const { return BT ? BK : (long long)BK * g.ldb; }

    // Fast path: the fragments of the first two sub-steps of slot SLOT, as the
    // last two sub-steps of the K step before read them.
    template <int SLOT>
    __device__ __forceinline__ void reread_frags() {
        read_frags<SLOT>(0, 0);
        read_frags<SLOT>(1, 1);
    }

    // Fast path: the loads of slices p0 (slot 0) and p1 (slot 1), nothing waited for.
    __device__ __forceinline__ void prologue_loads(const Next& p0, const Next& p1) {
        dma_b<0>(p0.n0, p0.kb, -1);
        dma_a<0>(p0.m0, p0.ka, -1);
        dma_b<1>(p1.n0, p1.kb, p1.vb);
        dma_a<1>(p1.m0, p1.ka, p1.va);
    }
    // Loads of one slice, per wave.
    static constexpr int NLD = A_DMA_N + B_DMA_N;

    // Store class of the tile at (m0, n0): 1 if each wave's epilogue issues at least
    // NST store instructions, else 0 (nothing counted).  The unmasked epilogue
    // issues exactly NST.  The masked one issues at least one store per 16-byte
    // chunk on a tile inside M x N (the pieces of a chunk that C's alignment calls
    // for are merged back into one store by the compiler, so no more are counted),
    // and a varying number on an edge tile.
    __device__ __forceinline__ int store_class(int m0, int n0) const {
        if constexpr (!EDGES)
            return 1;
        else
            return (m0 + BM <= g.M && n0 + BN <= g.N) ? 1 : 0;
    }
    // Barrier after a wait that lets the last EXTRA + sc * NST VMEM operations of
    // this wave stay in flight: EXTRA loads issued after the ones waited for, then
    // the epilogue stores of a tile of store class sc.
    template <int EXTRA>
    __device__ __forceinline__ void barrier_behind_stores(int sc) {
        constexpr int W = EXTRA + NST < 63 ? EXTRA + NST : 63;
        if (sc)
            barrier_after_loads<W>();
        else
            barrier_after_loads<EXTRA>();
    }

    // Prologue: slice p0 in slot 0 with the fragments of its first sub-step read
    // (fast path: of its first two); the fast path also has slice p1 in flight
    // into slot 1.  The first K step then loads the slices after.
    __device__ __forceinline__ void prologue(const Next& p0, const Next& p1) {
        if constexpr (FAST) {
            dma_b<0>(p0.n0, p0.kb, -1);
            dma_a<0>(p0.m0, p0.ka, -1);
            dma_b<1>(p1.n0, p1.kb, p1.vb);
            dma_a<1>(p1.m0, p1.ka, p1.va);
            barrier_after_loads<B_DMA_N + A_DMA_N>();
            read_frags<0>(0, 0);
            read_frags<0>(1, 1);
            return;
        } else {
            load_b<0>(p0.n0, p0.kb, -1);
            load_a(p0.m0, p0.ka, -1);
            store_a<0>();
            store_b<0, 0>();
            __syncthreads();
        }
        read_frags<0>(0, 0);
    }

    // End of the program: the direct-to-LDS loads of slices past the last one are
    // still in flight after the last barrier; let them land before the waves end
    // and the workgroup's LDS is handed to another.
    __device__ __forceinline__ void drain() {
        if (FAST) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // Full pipeline over K steps [k0, k1) of one tile (no epilogue): steps alternate
    // B slots 0 and 1; an odd step count runs one slot-0 step first and then pairs
    // starting on slot 1.
    template <bool RFL = false>
    __device__ __forceinline__ void tile_mainloop(int m0, int n0, int k0, int k1) {
        prologue(Next{m0, k0, -1, n0, k0, -1},
                 Next{m0, k0 + 1, vmask<RFL>(k0 + 1, k1), n0, k0 + 1, vmask<RFL>(k0 + 1, k1)});
        auto nx = [&](int k) {  // loads of step k
            return Next{m0, k + DA, vmask<RFL>(k + DA, k1), n0, k + DB, vmask<RFL>(k + DB, k1)};
        };
        int k = k0;
        if ((k1 - k0) & 1) {
            kstep<0>(nx(k0));
            for (k = k0 + 1; k < k1; k += 2) {
                kstep<1>(nx(k));
                kstep<0>(nx(k + 1));
            }
        } else {
            for (; k < k1; k += 2) {
                kstep<0>(nx(k));
                kstep<1>(nx(k + 1));
            }
        }
    }

    // Stream-K partial tile: the fp32 accumulators in register order, threads
    // interleaved -- float4 number u = (i * FN + j) * 4 + q of thread tid (its
    // accumulator block (i, j), values 4q .. 4q + 3) at index u * NT + tid -- so
    // that every store and load of a wave moves 1 KiB of consecutive bytes and the
    // owner of the tile reads back exactly the values its own registers hold.
    // Partial tiles move between XCDs, whose L2s are not coherent with each other:
    // they are written and read with device-scope cache policy (sc1: written through
    // the L2 and read past it), like the device-scope atomics, so that publishing
    // one needs only the writes to complete, not a write-back of the whole L2.
    // Buffer accesses: the per-lane offset is the same for every access and the
    // block offset goes in the scalar offset, so that no per-access address
    // registers are needed beside the accumulators.
    static constexpr int PART_FLOATS = BM * BN;
    static constexpr int kDeviceScope = 16;   // cache policy bit sc1
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float* part) const {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(part), (short)0, PART_FLOATS * 4, kBufferFlags);
    }
    __device__ __forceinline__ void write_partial(float* part) const {
        const __amdgpu_buffer_rsrc_t r = part_rsrc(part);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // whole-vector casts only: a bit cast of one element of a vector
                    // value is not reliable in this compiler (it reads element 0)
                    const f32x4 f = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f), r, tid * 16,
                                                           ((i * FN + j) * 4 + q) * NT * 16, kDeviceScope);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    // Partial tiles first .. last of a split tile, added in the epilogue (the
    // accumulators themselves are not changed, which keeps them in place).
    struct Parts {
        const float* base;   // partial tile 0
        int first, last;     // none if first > last
    };
    // v[0..3] (float4 number u of this thread) += partial tiles first .. last, in
    // order; two partial tiles' loads are in flight at a time.
    __device__ __forceinline__ void add_parts(float* v, const Parts& pt, int u, int t) const {
        int c = pt.first;
        for (; c + 1 <= pt.last; c += 2) {
            const f32x4 p0 = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(part_rsrc(pt.base + (long long)c * PART_FLOATS), t * 16,
                                                             u * NT * 16, kDeviceScope));
            const f32x4 p1 = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(part_rsrc(pt.base + (long long)(c + 1) * PART_FLOATS),
                                                             t * 16, u * NT * 16, kDeviceScope));
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (v[e] + p0[e]) + p1[e];
        }
        if (c <= pt.last) {
            const f32x4 p = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(part_rsrc(pt.base + (long long)c * PART_FLOATS), t * 16,
                                                             u * NT * 16, kDeviceScope));
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += p[e];
        }
    }

    // Epilogue of the BK = 64 tiles (fast and masked): each wave converts RS rows of its sub-tile at a time into
    // its own 4 KiB of LDS ([row][TN] of the output type, 16-byte chunks XOR-
    // swizzled by row so that the column writes and the row reads are free of bank
    // conflicts) and writes them back to C as whole row segments: lane l of a
    // 16-byte store covers chunk l mod CPR of row l / CPR, so a store instruction
    // writes 1 KiB of complete rows.  Lanes of a 32-row block whose row is not in
    // the current group skip the LDS write.  The masked kernels skip rows past M,
    // write the columns before N of a chunk that crosses N one by one, and split
    // whole chunks into pieces of the alignment C's rows allow.
    typedef typename Out<TO>::T OutT;
    static constexpr int OSZ = sizeof(OutT);
    static constexpr int ROWB = Cfg::TN * OSZ;                  // bytes of one sub-tile row
    static constexpr int CPR = ROWB / 16;                       // 16-byte chunks per row
    static constexpr int RS = Cfg::STAGE_W / ROWB;              // rows per staging pass
    static constexpr int NST = FAST ? FM * (32 / RS) * (Cfg::STAGE_W / 1024) : 0;  // stores per tile
    static constexpr bool STAGED = Cfg::C_BYTES > 0;
    static_assert(!STAGED || (RS >= 1 && 32 % RS == 0 && (CPR == 8 || CPR == 16 || CPR == 32 || CPR == 64)),
                  "staging shape");
    static_assert(!FAST || STAGED, "the fast path stages its epilogue");

    // One 16-byte chunk v of row segment p (its columns n .. n + 16/OSZ - 1, of which
    // `valid` are before N) to C, masked path.
    __device__ __forceinline__ void store_chunk_masked(char* p, const u32x4& v, int valid) const {
        constexpr int E = 16 / OSZ;
        if (valid >= E) {
            if (g.c_align >= 16) {
                *reinterpret_cast<u32x4*>(p) = v;
            } else if (g.c_align >= 8) {
                reinterpret_cast<u32x2*>(p)[0] = u32x2{v[0], v[1]};
                reinterpret_cast<u32x2*>(p)[1] = u32x2{v[2], v[3]};
            } else if (g.c_align >= 4) {
#pragma unroll
                for (int w = 0; w < 4; ++w) reinterpret_cast<uint32_t*>(p)[w] = v[w];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (e < valid) {
                    if (OSZ == 4)
                        reinterpret_cast<uint32_t*>(p)[e] = v[e];
                    else
                        reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    }
    static __device__ __forceinline__ int stage_swz(int r) { return (CPR == 8 ? (r >> 1) : r) & (CPR - 1); }

    template <bool PARTS>
    __device__ __forceinline__ void store_tile_staged(int m0, int n0, const Parts& pt) {
        // The lane index passes through an opaque copy here, so the per-lane
        // addresses below are formed at the store; otherwise, where the epilogue sits
        // inside a K loop, they are hoisted out of it and held in registers through
        // every step.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int tt = tid;
        if (PARTS) asm volatile("" : "+v"(tt));
        const int r32 = ln & 31, hk = ln >> 5;
        char* st = ldsc + wave * Cfg::STAGE_W;
        OutT* C = reinterpret_cast<OutT*>(g.C);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int h = 0; h < 32 / RS; ++h) {
                const int r = r32 - h * RS;   // row within this pass
                if (r >= 0 && r < RS) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            // columns 32 j + 8 q + 4 hk .. + 3 of row r
                            const int byte = (32 * j + 8 * q + 4 * hk) * OSZ;
                            const int ch = (byte >> 4) ^ stage_swz(r);
                            char* dst = st + r * ROWB + ch * 16 + (byte & 15);
                            float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                          acc[i][j][4 * q + 3]};
                            if (PARTS) add_parts(v, pt, (i * FN + j) * 4 + q, tt);
                            Out<TO>::store4(reinterpret_cast<OutT*>(dst), v, 4, true);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < Cfg::STAGE_W / 1024; ++u) {
                    const int off = u * 1024 + ln * 16;
                    const int row = off / ROWB, ch = (off % ROWB) >> 4;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(st + row * ROWB + ((ch ^ stage_swz(row)) << 4));
                    const long long m = m0 + wm * Cfg::TM + i * 32 + h * RS + row;
                    char* dst = reinterpret_cast<char*>(C + m * g.ldc + n0 + wn * Cfg::TN) + ch * 16;
                    if (!EDGES) {
                        *reinterpret_cast<u32x4*>(dst) = v;
                    } else if (m < g.M) {
                        store_chunk_masked(dst, v, g.N - (n0 + wn * Cfg::TN + ch * (16 / OSZ)));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Accumulators (plus, with PARTS, the partial tiles of pt) -> C (round to the
    // output type), masked to M x N.
    template <bool PARTS = false>
    __device__ __forceinline__ void store_tile(int m0, int n0, const Parts& pt = Parts{nullptr, 0, -1}) {
        if constexpr (STAGED) {
            store_tile_staged<PARTS>(m0, n0, pt);
            return;
        }
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
                    if (PARTS) add_parts(v, pt, (i * FN + j) * 4 + q, tid);
                    if (!MASKED) {
                        Out<TO>::store4(crow + n, v, 4, true);
                    } else {
                        const int valid = g.N - n;
                        if (valid > 0) Out<TO>::store4(crow + n, v, valid, g.vec_c);
                    }
                }
                // one block at a time: keeps the accumulator reads from being hoisted
                // into one burst that needs 256 more registers
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
};

// ---- kernels -------------------------------------------------------------------------

// Stream-K fix-up of a split tile (MODE_STREAMK; see StreamK).  The range holding
// K step 0 of a tile finishes it: it waits until every later range of the tile
// (r + 1 .. last) has published its partial tile, and its epilogue adds them to its
// own accumulators in range order (a fixed order, so the result is the same on
// every run) before storing C.  Any other piece publishes its accumulators as the
// range's partial tile -- device-scope writes, completed before the flag is set --
// and raises the range's flag; the finishing range clears the flag again, so the
// flags are zero between launches.  A range publishes before it waits for
// anything, and only ranges of lower program index are waited for, so the waits
// end once those programs run; a wait that exceeds sk_spin sleeps still gives up
// (counted in sk_err).
template <class E>
__device__ __forceinline__ void streamk_publish(E& e, const GemmArgs& g, int r) {
    e.write_partial(g.sk_part + (long long)r * E::PART_FLOATS);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // written through to device scope
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(g.sk_flags + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits for the flags of ranges r + 1 .. last and clears them; the partial tiles
// are then read (device scope) by the epilogue.
__device__ __forceinline__ void streamk_wait(const GemmArgs& g, int r, int last) {
    if (threadIdx.x == 0) {
        for (int c = r + 1; c <= last; ++c) {
            int n = 0;
            while (__hip_atomic_load(g.sk_flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                __builtin_amdgcn_s_sleep(2);
                if (++n > g.sk_spin) {
                    __hip_atomic_fetch_add(g.sk_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            __hip_atomic_store(g.sk_flags + c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
}

// Tiled, persistent and stream-K modes: for each of the program's work pieces, a
// full pipeline (prologue loads, K loop with two slices in flight, epilogue).  A
// piece is a whole tile, or in stream-K mode first the (at most two) pieces of
// the program's range of split tiles.  One loop runs every kind of piece, so the
// K loop is instantiated once.
template <class Cfg, class TI, class TO, int PATH, int MODE>
__global__ void __launch_bounds__(Cfg::NT) gemm_tiles_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char lds_a0[Cfg::A_SLOT], lds_a1[Cfg::A_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_b0[Cfg::B_SLOT], lds_b1[Cfg::B_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_c[Cfg::C_BYTES > 0 ? Cfg::C_BYTES : 16];
    typedef Engine<Cfg, TI, TO, PATH> E;
    E e(g, lds_a0, lds_a1, lds_b0, lds_b1, lds_c);
    ProgramClock pc;
    pc.start(g);
    const int ks = g.s.ks;
    // stream-K range of this program: items [b, end) of the split tiles
    int limit = g.s.num_tiles, r = 0, b = 0, end = 0;
    StreamK sk(g.s);
    if constexpr (MODE == MODE_STREAMK) {
        limit = sk.dp_tiles;
        r = sk.range_of_program(g.s, blockIdx.x);
        b = sk.range_begin(r);
        end = sk.range_begin(r + 1);
    }
    const ProgramWork w(g.s, blockIdx.x, limit);
    const int ntiles = (MODE == MODE_TILED) ? 1 : w.ntiles;
    for (int i = 0;;) {
        int tile, k0 = 0, k1 = ks;
        bool split = false;
        if (MODE == MODE_STREAMK && b < end) {
            const int t = b / ks;
            tile = sk.dp_tiles + t;
            k0 = b - t * ks;
            k1 = k0 + (end - b) < ks ? k0 + (end - b) : ks;
            split = k0 > 0 || k1 < ks;
            b += k1 - k0;
        } else if (i < ntiles) {
            tile = w.tile_id(i++);
        } else {
            break;
        }
        int tm, tn;
        tile_coords(g.s, tile, tm, tn);
        const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
        e.zero_acc();
        if (PATH != PATH_MASKED || ks > 0) e.template tile_mainloop<MODE == MODE_STREAMK>(m0, n0, k0, k1);
        if constexpr (MODE == MODE_STREAMK) {
            typename E::Parts pt{g.sk_part, r + 1, r};   // none
            if (split) {
                if (k0 > 0) {
                    streamk_publish(e, g, r);
                    continue;
                }
                pt.last = sk.range_of((tile - sk.dp_tiles + 1) * ks - 1);
                streamk_wait(g, r, pt.last);
            }
            e.template store_tile<true>(m0, n0, pt);
        } else {
            e.store_tile(m0, n0);
        }
    }
    e.drain();
    pc.stop(g);
}

// Position of the flattened loop: cursor plus the origin of its tile.
struct FlatPos {
    FlatCursor c;
    int m0, n0;
    template <class Cfg>
    __device__ __forceinline__ void coords(const SchedArgs& s) {
        int tm, tn;
        tile_coords(s, c.tile, tm, tn);
        m0 = tm * Cfg::BM;
        n0 = tn * Cfg::BN;
    }
    template <class Cfg>
    __device__ __forceinline__ void advance(const SchedArgs& s, const ProgramWork& w) {
        const int t = c.tile;
        c.advance(w);
        if (c.tile != t) coords<Cfg>(s);
    }
};

// Flattened cross-tile mode: one loop over (tile, k) items.  The slices of the
// next items -- the first slices of the next tile when item it ends a tile -- are
// in flight while item it is multiplied and, at a tile's last K step, stored.
template <class Cfg, class TI, class TO, int PATH>
__global__ void __launch_bounds__(Cfg::NT) gemm_flat_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char lds_a0[Cfg::A_SLOT], lds_a1[Cfg::A_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_b0[Cfg::B_SLOT], lds_b1[Cfg::B_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_c[Cfg::C_BYTES > 0 ? Cfg::C_BYTES : 16];
    typedef Engine<Cfg, TI, TO, PATH> E;
    E e(g, lds_a0, lds_a1, lds_b0, lds_b1, lds_c);
    ProgramClock pc;
    pc.start(g);
    const ProgramWork w(g.s, blockIdx.x);
    const int total = w.total_items();
    if (total == 0) {
        pc.stop(g);
        return;
    }
    // Two K steps per tile: the product is nearly all C write, and programs that
    // start together store their tiles together.  Groups of eight consecutive
    // programs start 2048 cycles apart, which spreads the bursts over one tile's
    // time (measured at 16384^2 x 128: 5-11 % faster; at 3 to 6 K steps, or with
    // fewer than 8 tiles per program, no faster or slower, so not there).
    if (w.ksp == 2 && w.ntiles >= 8) {
        const int grp = (blockIdx.x >> 3) & 7;
        for (int i = 0; i < grp; ++i) __builtin_amdgcn_s_sleep(32);
    }
    FlatPos cp{FlatCursor(w), 0, 0};   // item being multiplied
    cp.template coords<Cfg>(g.s);
    FlatPos p1 = cp;                   // item 1
    p1.template advance<Cfg>(g.s, w);
    e.prologue(typename E::Next{cp.m0, cp.c.k, -1, cp.n0, cp.c.k, -1},
               typename E::Next{p1.m0, p1.c.k, E::vmask(1, total), p1.n0, p1.c.k, E::vmask(1, total)});
    FlatPos ld = p1;                   // next item whose slices are loaded (DA = DB ahead)
    static_assert(E::DA == E::DB, "one load cursor");
    if (E::DA == 2) ld.template advance<Cfg>(g.s, w);
    // cursors past the program's last item get tile (0, 0) from tile_coords; nothing
    // is loaded (record count 0) or stored for them

    int it = 0;
    bool stored = false;               // the item before ended a tile (its stores are in flight)
    auto step = [&](auto slot_tag) {
        constexpr int SLOT = decltype(slot_tag)::value;
        if (cp.c.k == 0) e.zero_acc();
        const int vm = E::vmask(it + E::DA, total);
        e.template kstep<SLOT>(typename E::Next{ld.m0, ld.c.k, vm, ld.n0, ld.c.k, vm}, stored);
        ld.template advance<Cfg>(g.s, w);
        stored = cp.c.last_k(w);
        if (stored) {
            e.store_tile(cp.m0, cp.n0);
            // fast path: the fragments the step read ahead are dropped and read
            // again after the epilogue, which then runs with none of them held
            if constexpr (E::FAST) e.template reread_frags<SLOT ^ 1>();
        }
        cp.template advance<Cfg>(g.s, w);
        ++it;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (total & 1) {
        step(S0{});
        while (it < total) {
            step(S1{});
            step(S0{});
        }
    } else {
        while (it < total) {
            step(S0{});
            step(S1{});
        }
    }
    e.drain();
    pc.stop(g);
}

// Cross-tile mode on the direct-to-LDS tiles with at least two K steps per tile:
// the same (tile, k) sequence as the flattened loop, run as a loop over the
// program's tiles with the K loop inside, so that the per-step work has no cursor
// to advance.  The loads stay two items ahead, so the last two K
// steps of a tile load the first two slices of the next one, and those are in
// flight while the tile is stored.  The last K step of a tile does not wait for
// the next slice at its barrier (the fragments it reads ahead are read again);
// that wait comes after the epilogue, where this tile's stores, issued after the
// loads it waits for, may stay in flight: a wave then waits only for the stores
// of the tile before, one tile earlier, instead of those it has just issued
// (loads and stores retire in issue order on one counter).
// DEFER false (programs of more than one tile): the last K step of a tile waits for
// the next slice at its own barrier, as in the flattened loop, and after the
// epilogue the next tile only reads its first fragments again, with no barrier: two
// barriers a tile instead of three, and with the fragments read after the epilogue
// nothing but the accumulators is live through it, so the loop needs no spills (the
// flattened loop spills).
template <class Cfg, class TI, class TO, int PATH, bool DEFER = true>
__global__ void __launch_bounds__(Cfg::NT) gemm_xtile_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char lds_a0[Cfg::A_SLOT], lds_a1[Cfg::A_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_b0[Cfg::B_SLOT], lds_b1[Cfg::B_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_c[Cfg::C_BYTES > 0 ? Cfg::C_BYTES : 16];
    typedef Engine<Cfg, TI, TO, PATH> E;
    static_assert(E::FAST && E::DA == 2 && E::DB == 2, "direct-to-LDS pipeline, two slices ahead");
    E e(g, lds_a0, lds_a1, lds_b0, lds_b1, lds_c);
    ProgramClock pc;
    pc.start(g);
    const ProgramWork w(g.s, blockIdx.x);
    const int nt = w.ntiles, ks = w.ksp;
    if (nt == 0) {
        pc.stop(g);
        return;
    }
    int m0, n0, m1 = 0, n1 = 0;   // this tile and the next
    int sc = 0;                   // store class of the tile before
    {
        int tm, tn;
        tile_coords(g.s, w.tile_id(0), tm, tn);
        m0 = tm * Cfg::BM;
        n0 = tn * Cfg::BN;
        if (nt > 1) {
            tile_coords(g.s, w.tile_id(1), tm, tn);
            m1 = tm * Cfg::BM;
            n1 = tn * Cfg::BN;
        }
    }
    // two K steps a tile: the staggered start of the flattened loop (see there), from
    // 16 tiles per program (interleaved at K = 128: 16384^2, 16 tiles, 5.6-8.7 %
    // faster; 16384 x 8192 and 12288 x 16384, 8 and 12 tiles, 4-5 % slower)
    if (!DEFER && ks == 2 && nt >= 16) {
        const int grp = (blockIdx.x >> 3) & 7;
        for (int i = 0; i < grp; ++i) __builtin_amdgcn_s_sleep(32);
    }
    e.prologue_loads(typename E::Next{m0, 0, -1, n0, 0, -1}, typename E::Next{m0, 1, -1, n0, 1, -1});
    if constexpr (!DEFER) e.template barrier_after_loads<E::NLD>();   // the first slice has landed
    const long long a_ks = e.a_kstride(), b_ks = e.b_kstride();
    // one tile: S0 is the slot of its first K step (item i * ks); ODD: ks is odd,
    // so the slots of consecutive tiles start alternately on 0 and 1
    auto run_tile = [&](int i, auto s0_tag, auto odd_tag) {
        constexpr int S0 = decltype(s0_tag)::value;
        constexpr bool ODD = decltype(odd_tag)::value;
        // K step k loads item (i, k + 2), in the next tile from k = ks - 2 on: its
        // slices' element offsets run on by one slice stride a step and jump to the
        // next tile's origin after step ks - 3, so no step multiplies
        const long long a_next = e.a_slice(m1, 0), b_next = e.b_slice(n1, 0);
        const int vn = E::vmask(i + 1, nt);   // -1 if there is a next tile, else 0
        const bool two = ks == 2;             // step 0 already loads the next tile
        long long a_ld = two ? a_next : e.a_slice(m0, 2), b_ld = two ? b_next : e.b_slice(n0, 2);
        int kl = two ? 0 : 2, vl = two ? vn : -1;   // slice index within its tile, record-count mask
        auto advance = [&](int k) {   // after step k: the loads of step k + 1
            if (k + 3 == ks) {
                a_ld = a_next;
                b_ld = b_next;
                kl = 0;
                vl = vn;
            } else {
                a_ld += a_ks;
                b_ld += b_ks;
                ++kl;
            }
        };
        // the first slice of this tile has landed; behind it are its second slice
        // and the stores of the tile before, which may stay in flight (DEFER false:
        // the last K step's barrier or the prologue has already waited for it)
        if constexpr (DEFER) e.template barrier_behind_stores<E::NLD>(sc);
        e.template reread_frags<S0>();
        e.zero_acc();
        e.template kstep_at<S0>(a_ld, b_ld, kl, vl, i > 0, sc);
        advance(0);
        // steps 1 .. ks - 2 in pairs (odd ks: the last of them alone), then the last
        const int kend = ODD ? ks - 2 : ks - 1;
        for (int k = 1; k < kend; k += 2) {
            e.template kstep_at<S0 ^ 1>(a_ld, b_ld, kl, vl, false, 0);
            advance(k);
            e.template kstep_at<S0>(a_ld, b_ld, kl, vl, false, 0);
            advance(k + 1);
        }
        if constexpr (ODD) {
            e.template kstep_at<S0 ^ 1>(a_ld, b_ld, kl, vl, false, 0);
            advance(ks - 2);
            e.template kstep_at<S0, DEFER>(a_ld, b_ld, kl, vl, false, 0);
        } else {
            e.template kstep_at<S0 ^ 1, DEFER>(a_ld, b_ld, kl, vl, false, 0);
        }
        e.store_tile(m0, n0);
        sc = e.store_class(m0, n0);
        m0 = m1;
        n0 = n1;
        if (i + 2 < nt) {
            int tm, tn;
            tile_coords(g.s, w.tile_id(i + 2), tm, tn);
            m1 = tm * Cfg::BM;
            n1 = tn * Cfg::BN;
        }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using Even = std::integral_constant<bool, false>;
    using Odd = std::integral_constant<bool, true>;
    if (ks & 1) {
        for (int i = 0; i < nt; ++i) {
            if (i & 1)
                run_tile(i, C1{}, Odd{});
            else
                run_tile(i, C0{}, Odd{});
        }
    } else {
        for (int i = 0; i < nt; ++i) run_tile(i, C0{}, Even{});
    }
    e.drain();
    pc.stop(g);
}

// Schedule trace: one thread per program, the same functions as above.
__global__ void trace_kernel(SchedArgs s, int mode, int max_items, int32_t* out);

}  // namespace ts
