// Kernel instances of the ping-pong configuration on the zero-filled-edge path
// (stream-K uses the 8-wave kernels of the same tile).
#include "pingpong.hpp"

namespace ts {
KernelRef kernels_cfg256pp_edge(int io, int path, int mode) {
    if (mode == MODE_STREAMK) return kernels_cfg256w8_edge(io, path, mode);
    return pingpong_for<Cfg256w8, true>(io, PATH_EDGE);
}
}  // namespace ts
