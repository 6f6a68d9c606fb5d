// Kernel instances of the 64-wide tile configuration (every mode, type pair and
// masking variant).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg64(int io, bool masked, int mode) { return kernel_for<Cfg64>(io, masked, mode); }
}  // namespace ts
