// Kernel instances of the 256x256x64 tile configuration with 8 waves (two per
// SIMD, 128x64 per wave), every mode, type pair and path.
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256w8(int io, int path, int mode) { return kernel_for<Cfg256w8, KG_BASE>(io, path, mode); }
}  // namespace ts
