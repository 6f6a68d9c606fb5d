// Ping-pong GEMM kernel for gfx950: the 8-wave tile of gemm_kernel.hpp (same
// LDS layout, loads, fragment reads, MFMAs and epilogue, taken from its Engine)
// with the waves split into two groups that take turns at the matrix units.
//
// What is computed is the same as the other kernels: each program walks its
// tiles in the order of the tiled, persistent or flattened loop of "(1/n) Triton
// matmul ... persistent kernel" and "(3/n) ... cross tile pipelining" (one fp32
// accumulator per tile, reset at the tile's first K step), and every accumulator
// takes its K sub-steps in the same order, so the output is bit for bit that of
// the 8-wave kernel.  How it is scheduled is this file's own design.
#pragma once

#include "internal.hpp"

namespace ts {
namespace pp {

// Buffer resources of slice k of tile (m0, n0); `valid` 0 turns every load of the
// slice into zeros with no memory access (items past the program's last one).
// Edge paths: also sets the k limit of the slice's A chunks.
template <class E>
struct Slice {
    __amdgpu_buffer_rsrc_t ra, rb;
};
template <class E>
__device__ __forceinline__ Slice<E> slice_rsrc(E& e, int m0, int n0, int k, int valid = -1) {
    if constexpr (E::EDGE) e.klim = e.g.K - k * E::BK;
    return Slice<E>{e.rsrc_a(e.a_slice(m0, k), valid), e.rsrc_b(e.b_slice(n0, k), valid)};
}

// This wave's load number c (B loads first, then A) of a slice into slot SLOT.
template <int SLOT, class E>
__device__ __forceinline__ void dma_one(E& e, int c, const Slice<E>& sl) {
    if (c < E::B_DMA_N)
        e.template dma_b_one<SLOT>(c, sl.rb);
    else
        e.template dma_a_one<SLOT>(c - E::B_DMA_N, sl.ra);
}
template <int SLOT, class E>
__device__ __forceinline__ void dma_all(E& e, const Slice<E>& sl) {
#pragma unroll
    for (int c = 0; c < E::NVM; ++c) dma_one<SLOT>(e, c, sl);
}

// The MFMAs of two sub-steps (fragment buffers 0 and 1).  With LOAD, this wave's
// loads of slice sl into slot SLOT go out between them, one every other MFMA.
template <bool LOAD, int SLOT, class E>
__device__ __forceinline__ void mma_pair(E& e, const Slice<E>& sl) {
    static_assert(E::NMF >= E::NVM, "one load per two MFMAs");
#pragma unroll
    for (int t = 0; t < 2 * E::NMF; ++t) {
        e.mfma_one(t / E::NMF, t % E::NMF);
        if (LOAD && (t & 1) == 0 && t / 2 < E::NVM) dma_one<SLOT>(e, t / 2, sl);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The fragments of sub-steps s0 and s0 + 1 of slot SLOT into buffers 0 and 1.
template <int SLOT, class E>
__device__ __forceinline__ void read_pair(E& e, int s0) {
    e.template read_frags<SLOT>(s0, 0);
    e.template read_frags<SLOT>(s0 + 1, 1);
}

// End of a phase: this wave's LDS reads are done and, for VM >= 0, all but its
// last VM memory operations; then the workgroup meets.
template <int VM>
__device__ __forceinline__ void phase_end() {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (VM < 0)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace pp

// Ping-pong kernel (8 waves, direct-to-LDS paths).  The waves form two groups of
// four -- waves 0-3 own tile rows 0..BM/2-1, waves 4-7 the rest -- which the
// dispatcher places one of each per SIMD.  Each K step is four phases separated by
// workgroup barriers; in every phase one group runs the MFMAs of two sub-steps from
// fragments already in its registers while the other group reads its next two
// sub-steps' fragments from LDS, so the matrix unit of each SIMD is fed by one wave
// at a time and neither waits for the other's LDS traffic:
//
//   phase   leading group (waves 0-3)            trailing group (waves 4-7)
//   1       MFMA sub-steps 0-1 of item it         read 0-1 of it
//   2       read 2-3 of it                       MFMA 0-1 of it
//   3       MFMA 2-3 of it                       read 2-3 of it
//   4       loads of item it + 2; read 0-1 of    MFMA 2-3 of it, loads of item it + 2
//           item it + 1
//
// An item is one (tile, K step) of the program's tiles taken in order (the tiled,
// persistent and cross-tile maps of the other kernels), so the tile boundary does
// not drain the pipeline: each group stores a finished tile in the next phase in
// which it reads (the leading group in phase 4, the trailing group in phase 1 of
// the next tile's first item) and starts the next tile with cleared accumulators.
// Slot it mod 2 holds item it; every read of it ends in phase 3, so phase 4 can
// load item it + 2 into it, and each wave waits for its own loads of item it + 1
// at the end of phase 3, before anyone reads them.
template <class Cfg, class TI, class TO, int PATH>
__global__ void __launch_bounds__(Cfg::NT) gemm_pingpong_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char lds_a0[Cfg::A_SLOT], lds_a1[Cfg::A_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_b0[Cfg::B_SLOT], lds_b1[Cfg::B_SLOT];
    __shared__ __attribute__((aligned(16))) char lds_c[Cfg::C_BYTES > 0 ? Cfg::C_BYTES : 16];
    typedef Engine<Cfg, TI, TO, PATH> E;
    static_assert(E::FAST && E::NW == 8 && Cfg::WM == 2 && E::SUB == 4, "two groups of four waves, BK = 64");
    // stores of a tile that may stay in flight at a wait for loads issued before them
    // (the edge paths issue a varying number and wait for all)
    constexpr int ST = E::EDGES ? 0 : (E::NST < 63 ? E::NST : 0);
    E e(g, lds_a0, lds_a1, lds_b0, lds_b1, lds_c);
    ProgramClock pc;
    pc.start(g);
    const ProgramWork w(g.s, blockIdx.x);
    const int total = w.total_items();
    if (total == 0) {
        pc.stop(g);
        return;
    }
    const bool lead = e.wave < E::NW / 2;
    e.zero_acc();
    FlatPos cp{FlatCursor(w), 0, 0};   // item being multiplied
    cp.template coords<Cfg>(g.s);
    FlatPos ld = cp;                   // next item to load
    {
        pp::Slice<E> sl = pp::slice_rsrc(e, ld.m0, ld.n0, ld.c.k);
        pp::dma_all<0>(e, sl);
        ld.template advance<Cfg>(g.s, w);
        if (total > 1) {
            sl = pp::slice_rsrc(e, ld.m0, ld.n0, ld.c.k);
            pp::dma_all<1>(e, sl);
        }
        ld.template advance<Cfg>(g.s, w);
    }
    if (total > 1)
        pp::phase_end<E::NVM>();
    else
        pp::phase_end<0>();
    if (lead) pp::read_pair<0>(e, 0);
    pp::phase_end<-1>();

    // Each group runs its own loop (the accumulators never meet at a branch merge);
    // both meet the same barriers, four per item.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    int it = 0;
    bool stored = false;   // this wave's tile stores went out after its loads of the next item
    if (lead) {
        auto item = [&](auto slot_tag) {
            constexpr int SLOT = decltype(slot_tag)::value;
            pp::mma_pair<false, SLOT>(e, pp::Slice<E>{});
            pp::phase_end<-1>();
            pp::read_pair<SLOT>(e, 2);
            pp::phase_end<-1>();
            pp::mma_pair<false, SLOT>(e, pp::Slice<E>{});
            if (stored)
                pp::phase_end<ST>();
            else
                pp::phase_end<0>();
            pp::dma_all<SLOT>(e, pp::slice_rsrc(e, ld.m0, ld.n0, ld.c.k, E::template vmask<false>(it + 2, total)));
            stored = false;
            if (cp.c.last_k(w)) {
                e.store_tile(cp.m0, cp.n0);
                e.zero_acc();
                stored = true;
            }
            pp::read_pair<SLOT ^ 1>(e, 0);
            pp::phase_end<-1>();
            ld.template advance<Cfg>(g.s, w);
            cp.template advance<Cfg>(g.s, w);
            ++it;
        };
        while (it < total) {
            item(S0{});
            if (it < total) item(S1{});
        }
    } else {
        int pm0 = cp.m0, pn0 = cp.n0;   // tile of the item before
        auto item = [&](auto slot_tag) {
            constexpr int SLOT = decltype(slot_tag)::value;
            stored = false;
            if (cp.c.k == 0 && it > 0) {
                e.store_tile(pm0, pn0);
                e.zero_acc();
                stored = true;
            }
            pp::read_pair<SLOT>(e, 0);
            pp::phase_end<-1>();
            pp::mma_pair<false, SLOT>(e, pp::Slice<E>{});
            pp::phase_end<-1>();
            pp::read_pair<SLOT>(e, 2);
            if (stored)
                pp::phase_end<ST>();
            else
                pp::phase_end<0>();
            pp::mma_pair<true, SLOT>(e, pp::slice_rsrc(e, ld.m0, ld.n0, ld.c.k, E::template vmask<false>(it + 2, total)));
            pp::phase_end<-1>();
            pm0 = cp.m0;
            pn0 = cp.n0;
            ld.template advance<Cfg>(g.s, w);
            cp.template advance<Cfg>(g.s, w);
            ++it;
        };
        while (it < total) {
            item(S0{});
            if (it < total) item(S1{});
        }
        e.store_tile(pm0, pn0);
    }
    e.drain();
    pc.stop(g);
}

// Ping-pong kernel of a direct-to-LDS path (PATH_FULL, PATH_FULL_BT or PATH_EDGE);
// every mode but stream-K runs it (its item stream covers the tiled, persistent and
// cross-tile maps).
template <class Cfg, int PATH>
const void* pingpong_by_io(int io) {
    switch (io) {
        case IO_F16_F16: return reinterpret_cast<const void*>(&gemm_pingpong_kernel<Cfg, InF16, OutF16, PATH>);
        case IO_F16_F32: return reinterpret_cast<const void*>(&gemm_pingpong_kernel<Cfg, InF16, OutF32, PATH>);
        case IO_BF16_BF16: return reinterpret_cast<const void*>(&gemm_pingpong_kernel<Cfg, InBF16, OutBF16, PATH>);
        default: return reinterpret_cast<const void*>(&gemm_pingpong_kernel<Cfg, InBF16, OutF32, PATH>);
    }
}
template <class Cfg, bool EDGE>
KernelRef pingpong_for(int io, int path) {
    const void* f = nullptr;
    if constexpr (EDGE)
        f = pingpong_by_io<Cfg, PATH_EDGE>(io);
    else
        f = path == PATH_FULL_BT ? pingpong_by_io<Cfg, PATH_FULL_BT>(io) : pingpong_by_io<Cfg, PATH_FULL>(io);
    return KernelRef{f, Cfg::NT, Cfg::LDS_BYTES};
}

}  // namespace ts
