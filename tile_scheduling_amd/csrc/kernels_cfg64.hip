// Kernel instances of the 64-wide tile configuration (every mode, type pair and
// path).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg64(int io, int path, int mode) { return kernel_for<Cfg64, KG_BASE>(io, path, mode); }
}  // namespace ts
