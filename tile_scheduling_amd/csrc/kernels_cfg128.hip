// Kernel instances of the 128-wide tile configuration (every mode, type pair and
// masking variant).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg128(int io, bool masked, int mode) { return kernel_for<Cfg128>(io, masked, mode); }
}  // namespace ts
