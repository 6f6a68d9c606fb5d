// Kernel instances of the ping-pong configuration: the 256x256x64 tile with 8
// waves (128x64 per wave) in two alternating groups, whole-tile paths (B stored
// [K][N] or [N][K]).  The modes and paths the ping-pong loop does not run (stream-K,
// the masked register path) use the 8-wave kernels of the same tile.
#include "pingpong.hpp"

namespace ts {
KernelRef kernels_cfg256pp(int io, int path, int mode) {
    if (mode == MODE_STREAMK || (path != PATH_FULL && path != PATH_FULL_BT)) return kernels_cfg256w8(io, path, mode);
    return pingpong_for<Cfg256w8, false>(io, path);
}
}  // namespace ts
