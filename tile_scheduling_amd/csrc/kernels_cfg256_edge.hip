// Zero-filled-edge kernel instances of the 256 tile configuration (every mode
// and type pair).
#include "internal.hpp"

namespace ts {
KernelRef kernels_cfg256_edge(int io, int path, int mode) { return kernel_for<Cfg256, KG_EDGE>(io, path, mode); }
}  // namespace ts
