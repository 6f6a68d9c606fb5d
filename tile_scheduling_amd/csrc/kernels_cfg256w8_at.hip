// Kernel instances of the 256x256x64 tile configuration with 8 waves (128x64 per wave) with A stored [K][M]
// (B stored [K][N] or [N][K]): whole tiles, every mode and type pair.
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256w8_at(int io, int path, int mode) { return kernel_for<Cfg256w8, KG_AT>(io, path, mode); }
}  // namespace ts
