// Declarations shared by the kernel-instance files and the C-ABI implementation.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "gemm_kernel.hpp"

namespace ts {

// Input/output type pair of a kernel instance.
enum : int { IO_F16_F16 = 0, IO_F16_F32 = 1, IO_BF16_BF16 = 2, IO_BF16_F32 = 3 };

// Tile configurations (same numbering as TS_TILE_* in tsgemm.h).  CFG_256PP is the
// 8-wave 256 x 256 x 64 tile run by the ping-pong kernel.
enum : int { CFG_64 = 1, CFG_128 = 2, CFG_256 = 3, CFG_256W8 = 4, CFG_256PP = 5 };

typedef TileCfg<64, 64, 32, 2, 2> Cfg64;
typedef TileCfg<128, 128, 64, 2, 2> Cfg128;
typedef TileCfg<256, 256, 64, 2, 2> Cfg256;
typedef TileCfg<256, 256, 64, 2, 4> Cfg256w8;   // 8 waves: two per SIMD

struct KernelRef {
    const void* fn;  // __global__ function, launched with one GemmArgs argument
    int threads;
    int lds_bytes;   // static LDS of the instance
};

// Whether a configuration has a cross-tile (flattened loop) kernel.  The 4-wave
// 256 x 256 x 64 tile has none: its 256 accumulators per lane do not survive the
// flattened loop's branch merges without about a thousand spilled registers.
template <class Cfg>
constexpr bool has_flat_kernel() { return !std::is_same<Cfg, Cfg256>::value; }

template <class Cfg, class TI, class TO, int PATH>
const void* kernel_by_mode(int mode) {
    switch (mode) {
        case MODE_TILED: return reinterpret_cast<const void*>(&gemm_tiles_kernel<Cfg, TI, TO, PATH, MODE_TILED>);
        case MODE_PERSISTENT: return reinterpret_cast<const void*>(&gemm_tiles_kernel<Cfg, TI, TO, PATH, MODE_PERSISTENT>);
        case MODE_STREAMK: return reinterpret_cast<const void*>(&gemm_tiles_kernel<Cfg, TI, TO, PATH, MODE_STREAMK>);
        case MODE_XTILE:
            if constexpr (has_flat_kernel<Cfg>() && Engine<Cfg, TI, TO, PATH>::FAST)
                return reinterpret_cast<const void*>(&gemm_xtile_kernel<Cfg, TI, TO, PATH>);
            else
                return nullptr;
        case MODE_XTILE_PLAIN:
            if constexpr (has_flat_kernel<Cfg>() && Engine<Cfg, TI, TO, PATH>::FAST)
                return reinterpret_cast<const void*>(&gemm_xtile_kernel<Cfg, TI, TO, PATH, false>);
            else
                return nullptr;
        default:
            if constexpr (has_flat_kernel<Cfg>())
                return reinterpret_cast<const void*>(&gemm_flat_kernel<Cfg, TI, TO, PATH>);
            else
                return nullptr;
    }
}

// Whole-tile and masked-register instances (one translation unit per tile
// configuration) and zero-filled-edge instances (a second one), so that the
// configurations compile in parallel in halves.
template <class Cfg, class TI, class TO>
const void* kernel_by_path_base(int path, int mode) {
    if (path == PATH_FULL) return kernel_by_mode<Cfg, TI, TO, PATH_FULL>(mode);
    if (path == PATH_FULL_BT) {
        if constexpr (Engine<Cfg, TI, TO, PATH_FULL>::FAST_OK)
            return kernel_by_mode<Cfg, TI, TO, PATH_FULL_BT>(mode);
        else
            return nullptr;
    }
    return kernel_by_mode<Cfg, TI, TO, PATH_MASKED>(mode);
}
template <class Cfg, class TI, class TO>
const void* kernel_by_path_edge(int path, int mode) {
    static_assert(Engine<Cfg, TI, TO, PATH_FULL>::FAST_OK, "the edge path needs the direct-to-LDS pipeline");
    (void)path;
    return kernel_by_mode<Cfg, TI, TO, PATH_EDGE>(mode);
}

// Whole-tile instances with A stored [K][M] (B stored [K][N] or [N][K]): square
// direct-to-LDS tiles only.
template <class Cfg, class TI, class TO>
const void* kernel_by_path_at(int path, int mode) {
    if constexpr (Engine<Cfg, TI, TO, PATH_FULL>::FAST_OK && Cfg::BM == Cfg::BN) {
        if (path == PATH_FULL_ATBT) return kernel_by_mode<Cfg, TI, TO, PATH_FULL_ATBT>(mode);
        return kernel_by_mode<Cfg, TI, TO, PATH_FULL_AT>(mode);
    } else {
        (void)path;
        (void)mode;
        return nullptr;
    }
}

// Instance groups, one per translation unit of a tile configuration.
enum : int { KG_BASE = 0, KG_EDGE = 1, KG_AT = 2 };

template <class Cfg, class TI, class TO, int KG>
const void* kernel_by_path(int path, int mode) {
    if constexpr (KG == KG_EDGE)
        return kernel_by_path_edge<Cfg, TI, TO>(path, mode);
    else if constexpr (KG == KG_AT)
        return kernel_by_path_at<Cfg, TI, TO>(path, mode);
    else
        return kernel_by_path_base<Cfg, TI, TO>(path, mode);
}

template <class Cfg, int KG>
KernelRef kernel_for(int io, int path, int mode) {
    const void* f = nullptr;
    switch (io) {
        case IO_F16_F16: f = kernel_by_path<Cfg, InF16, OutF16, KG>(path, mode); break;
        case IO_F16_F32: f = kernel_by_path<Cfg, InF16, OutF32, KG>(path, mode); break;
        case IO_BF16_BF16: f = kernel_by_path<Cfg, InBF16, OutBF16, KG>(path, mode); break;
        default: f = kernel_by_path<Cfg, InBF16, OutF32, KG>(path, mode); break;
    }
    return KernelRef{f, Cfg::NT, Cfg::LDS_BYTES};
}

// Whether a configuration has the direct-to-LDS pipeline (and so the edge paths).
template <class Cfg>
constexpr bool has_fast_path() { return Engine<Cfg, InF16, OutF16, PATH_FULL>::FAST_OK; }
// Whether it has the whole-tile paths with A stored [K][M].
template <class Cfg>
constexpr bool has_at_path() { return has_fast_path<Cfg>() && Cfg::BM == Cfg::BN; }

// One function per tile configuration, each defined in its own translation unit.
// path PATH_FULL, PATH_FULL_BT or PATH_MASKED
KernelRef kernels_cfg64(int io, int path, int mode);
KernelRef kernels_cfg128(int io, int path, int mode);
KernelRef kernels_cfg256(int io, int path, int mode);
KernelRef kernels_cfg256w8(int io, int path, int mode);
KernelRef kernels_cfg256pp(int io, int path, int mode);
// path PATH_FULL_AT or PATH_FULL_ATBT (square direct-to-LDS configurations)
KernelRef kernels_cfg128_at(int io, int path, int mode);
KernelRef kernels_cfg256_at(int io, int path, int mode);
KernelRef kernels_cfg256w8_at(int io, int path, int mode);
// path PATH_EDGE (configurations with the direct-to-LDS pipeline)
KernelRef kernels_cfg128_edge(int io, int path, int mode);
KernelRef kernels_cfg256_edge(int io, int path, int mode);
KernelRef kernels_cfg256w8_edge(int io, int path, int mode);
KernelRef kernels_cfg256pp_edge(int io, int path, int mode);

}  // namespace ts
