// Kernel instances of the 256x256x64 tile configuration with 4 waves (128x128 per wave) with A stored [K][M]
// (B stored [K][N] or [N][K]): whole tiles, every mode and type pair.
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256_at(int io, int path, int mode) { return kernel_for<Cfg256, KG_AT>(io, path, mode); }
}  // namespace ts
