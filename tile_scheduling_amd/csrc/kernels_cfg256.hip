// Kernel instances of the 256-wide tile configuration (every mode, type pair and
// masking variant).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256(int io, bool masked, int mode) { return kernel_for<Cfg256>(io, masked, mode); }
}  // namespace ts
