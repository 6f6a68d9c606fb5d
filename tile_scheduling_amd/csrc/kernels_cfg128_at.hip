// Kernel instances of the 128x128x64 tile configuration (4 waves) with A stored [K][M]
// (B stored [K][N] or [N][K]): whole tiles, every mode and type pair.
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg128_at(int io, int path, int mode) { return kernel_for<Cfg128, KG_AT>(io, path, mode); }
}  // namespace ts
