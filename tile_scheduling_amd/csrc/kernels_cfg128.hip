// Kernel instances of the 128-wide tile configuration (every mode, type pair and
// path).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg128(int io, int path, int mode) { return kernel_for<Cfg128, KG_BASE>(io, path, mode); }
}  // namespace ts
