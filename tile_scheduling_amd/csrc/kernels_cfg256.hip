// Kernel instances of the 256-wide tile configuration (every mode, type pair and
// path).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256(int io, int path, int mode) { return kernel_for<Cfg256, KG_BASE>(io, path, mode); }
}  // namespace ts
