// C-ABI of the tiled GEMM library: argument validation, launch planning (tile
// configuration, grid, masking), dispatch to the kernel instances, and the
// schedule trace.  See include/tsgemm.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <dlfcn.h>
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/tsgemm.h"
#include "internal.hpp"
#include "resource_table.hpp"

namespace ts {

// Scratch memory of ts_gemm_noalloc: the stream-K workspace for callers that cannot
// allocate.  One copy per GPU, held until the process ends.  Host code never uses
// this name as an address: the device address comes from hipGetSymbolAddress,
// once per device (scratch_ptr below).
constexpr int64_t kScratchBytes = (64ll << 20) + (64 << 10);
static __device__ __align__(256) char scratch[kScratchBytes];

// Sets n words at p to zero (the flags of a stream-K workspace).
__global__ void clear_words(int* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void trace_kernel(SchedArgs s, int mode, int max_items, int32_t* out) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p < s.grid) trace_program(s, mode, p, max_items, out + (long long)p * max_items * 5);
}

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int cu_count = 0;
    int xcds = 8;
};

std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];          // device address of `scratch` on each device
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's copy of `scratch` (dev must be current).
ts_status scratch_ptr(int dev, void** out) {
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (g_scratch_err[dev] != hipSuccess) (void)hipGetLastError();
        g_scratch[dev] = ptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch[dev]) return TS_ERR_HIP;
    *out = g_scratch[dev];
    return TS_OK;
}

// Properties of the current device, queried once per device.
ts_status current_device(int* dev_out, DeviceInfo* info) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return TS_ERR_NO_DEVICE;
    }
    std::call_once(g_dev_once[dev], [dev]() {
        int cus = 0, x = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x < 1 || x > 64) x = 8;
        (void)hipGetLastError();
        g_dev[dev].cu_count = cus;
        g_dev[dev].xcds = x;
    });
    if (g_dev[dev].cu_count <= 0) return TS_ERR_NO_DEVICE;
    *dev_out = dev;
    *info = g_dev[dev];
    return TS_OK;
}

struct Plan {
    bool auto_order;        // TS_ORDER_AUTO: order, G and remap chosen in resolve_grid
    int l2_reuse_pm;        // the locality model's reuse of the resolved order (1/1000)
    int cfg;                // CFG_*
    int bm, bn, bk;
    int io;                 // IO_*
    int mode;
    bool masked;            // the tiles do not cover M x N x K exactly, or rows defeat 16-byte access
    int path;               // PATH_*: which kernel runs a masked plan
    int vec_a, vec_b, vec_c;
    SchedArgs s;            // grid filled once the device is known (persistent auto)
    int requested_programs; // 0 = auto
    int64_t max_items;
};

void cfg_dims(int cfg, int* bm, int* bn, int* bk) {
    switch (cfg) {
        case CFG_64: *bm = Cfg64::BM; *bn = Cfg64::BN; *bk = Cfg64::BK; break;
        case CFG_128: *bm = Cfg128::BM; *bn = Cfg128::BN; *bk = Cfg128::BK; break;
        case CFG_256W8:
        case CFG_256PP: *bm = Cfg256w8::BM; *bn = Cfg256w8::BN; *bk = Cfg256w8::BK; break;
        default: *bm = Cfg256::BM; *bn = Cfg256::BN; *bk = Cfg256::BK; break;
    }
}

// The nested cross-tile kernels run on the 128 x 128 and 8-wave 256 x 256
// direct-to-LDS tiles.  The one with the deferred wait (MODE_XTILE) needs at least
// this many K steps a tile: with fewer, its epilogues come so close together that
// the deeper queue of stores slows the loads behind them (measured on the 16384^2
// product: 9-10 % slower than the flattened loop at 2 steps, 2-4 % at 4 and 6,
// level at 8); it runs where a program has one tile (below).  TS_MODE_AUTO takes
// the cross-tile mode wherever a tile has at least this many steps on these tiles.
constexpr int kXtileMinSteps = 8;
bool xtile_shape(int cfg, int64_t ks) {
    return (cfg == CFG_128 || cfg == CFG_256W8) && ks >= kXtileMinSteps;
}

// The nested kernel without the deferred wait (MODE_XTILE_PLAIN) runs the
// cross-tile mode on the same tiles from 2 K steps on when a program has more than
// one tile (before the grid is resolved: always): two barriers a tile as in the
// flattened loop, but no spills where the flattened loop spills.  Measured on the
// 16384^2 product, interleaved: against the flattened loop, fp32 output 21 % faster
// at K = 128 and 11 % at K = 256 with bf16 inputs, fp16 3 % at K = 128 and 256,
// level from 5 to 7 steps, 2.5 % slower at 3; against the nested kernel with the
// deferred wait, 2.6 % faster at K = 512, 1.4 % at 1024, 0.3 % at 4096 and 1-1.5 %
// on the 5000 x 12290 x 1000 product.  With one tile per program there is no tile
// boundary to overlap: the flattened loop runs below 8 K steps (4096^2 at K = 256:
// 6 % faster than this kernel) and the deferred-wait kernel from 8 on.
bool xtile_plain_shape(const Plan& p) {
    return (p.cfg == CFG_128 || p.cfg == CFG_256W8) && p.s.ks >= 2 && (p.s.grid <= 0 || p.s.num_tiles > p.s.grid);
}

// Kernel mode of a plan: MODE_XTILE_PLAIN or MODE_XTILE where a nested cross-tile
// kernel runs, else the plan's own mode.
int kernel_mode(const Plan& p) {
    if (p.mode == TS_MODE_CROSSTILE && p.path != PATH_MASKED) {
        if (xtile_plain_shape(p)) return MODE_XTILE_PLAIN;
        if (xtile_shape(p.cfg, p.s.ks)) return MODE_XTILE;
    }
    return p.mode;
}

KernelRef kernel_of(const Plan& p) {
    const int km = kernel_mode(p);
    if (p.path == PATH_FULL_AT || p.path == PATH_FULL_ATBT) {   // only on square direct-to-LDS tiles
        switch (p.cfg) {
            case CFG_128: return kernels_cfg128_at(p.io, p.path, km);
            case CFG_256: return kernels_cfg256_at(p.io, p.path, km);
            default: return kernels_cfg256w8_at(p.io, p.path, km);   // the ping-pong tile runs these too
        }
    }
    const bool edge = p.path == PATH_EDGE;   // only on direct-to-LDS tiles
    switch (p.cfg) {
        case CFG_64: return kernels_cfg64(p.io, edge ? PATH_MASKED : p.path, km);
        case CFG_128: return edge ? kernels_cfg128_edge(p.io, p.path, km) : kernels_cfg128(p.io, p.path, km);
        case CFG_256W8: return edge ? kernels_cfg256w8_edge(p.io, p.path, km) : kernels_cfg256w8(p.io, p.path, km);
        case CFG_256PP: return edge ? kernels_cfg256pp_edge(p.io, p.path, km) : kernels_cfg256pp(p.io, p.path, km);
        default: return edge ? kernels_cfg256_edge(p.io, p.path, km) : kernels_cfg256(p.io, p.path, km);
    }
}

bool cfg_has_at_path(int cfg) {
    switch (cfg) {
        case CFG_64: return has_at_path<Cfg64>();
        case CFG_128: return has_at_path<Cfg128>();
        case CFG_256W8:
        case CFG_256PP: return has_at_path<Cfg256w8>();
        default: return has_at_path<Cfg256>();
    }
}

bool cfg_has_fast_path(int cfg) {
    switch (cfg) {
        case CFG_64: return has_fast_path<Cfg64>();
        case CFG_128: return has_fast_path<Cfg128>();
        case CFG_256W8:
        case CFG_256PP: return has_fast_path<Cfg256w8>();
        default: return has_fast_path<Cfg256>();
    }
}

// Kernel path of a plan.  A masked plan runs the direct-to-LDS pipeline with
// zero-filled edges when A's base is 16-byte aligned with K and its row stride
// multiples of 8 elements (a 16-byte chunk of A never mixes the end of a row
// with the next row), B's base is 4-byte aligned with N and its row stride even
// (no dword straddles the end of B), and the in-tile offsets stay below 2^30
// bytes.  Otherwise the masked register pipeline runs.
int choose_path(const Plan& p, int64_t N, int64_t K, uintptr_t a, uintptr_t b, int64_t lda, int64_t ldb) {
    if (!p.masked) return PATH_FULL;
    if (!cfg_has_fast_path(p.cfg) || K <= 0 || K % 8 != 0) return PATH_MASKED;
    if (a % 16 != 0 || lda % 8 != 0) return PATH_MASKED;
    if ((int64_t)p.bm * lda * 2 >= (1LL << 30) || (int64_t)p.bk * ldb * 2 >= (1LL << 30)) return PATH_MASKED;
    if (b % 4 == 0 && ldb % 2 == 0 && N % 2 == 0) return PATH_EDGE;
    return PATH_MASKED;
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// TS_MODE_AUTO: the cross-tile loop for tiles of at most this many K steps (at
// 16384^2 it leads the persistent loop by 2-17 % from K = 128 to 2048 and trails
// it by 1-1.5 % at K = 4096).
constexpr int64_t kCrossTileMaxSteps = 32;

// Locality model of a schedule: the first `concurrent` workgroups of the launch
// (the ones resident together; workgroup w runs on XCD w mod X) and the tiles they
// start on.  Each XCD's L2 serves the A row panels and B column panels its tiles
// share, so the cost is the number of distinct (XCD, tile row) plus (XCD, tile
// column) pairs; the reuse fraction is 1 - cost / (2 x tiles).
void locality_cost(const SchedArgs& s0, int concurrent, int64_t* cost, int64_t* tiles) {
    SchedArgs s = s0;
    s.fastdiv = 0;
    std::vector<int64_t> rows, cols;
    const int n = concurrent < s.grid ? concurrent : s.grid;
    for (int w = 0; w < n; ++w) {
        const int start = s.remap ? xcd_remap(w, s.grid, s.xcds) : w;
        if (start >= s.num_tiles) continue;
        int tm, tn;
        tile_coords(s, start, tm, tn);
        const int64_t x = w % s.xcds;
        rows.push_back((x << 32) | tm);
        cols.push_back((x << 32) | tn);
    }
    std::sort(rows.begin(), rows.end());
    std::sort(cols.begin(), cols.end());
    *tiles = (int64_t)rows.size();
    *cost = (int64_t)(std::unique(rows.begin(), rows.end()) - rows.begin()) +
            (int64_t)(std::unique(cols.begin(), cols.end()) - cols.begin());
}

// TS_ORDER_AUTO: the candidate of least locality cost, ties to the earlier one.
void choose_order(SchedArgs* s, int concurrent, int* reuse_pm) {
    struct Cand { int order, G, remap; };
    static const Cand kCands[] = {{ORDER_GROUPED, 8, 1},  {ORDER_GROUPED, 4, 1},  {ORDER_GROUPED, 16, 1},
                                  {ORDER_ROW_MAJOR, 1, 0}, {ORDER_ROW_MAJOR, 1, 1}, {ORDER_GROUPED, 8, 0},
                                  {ORDER_GROUPED, 4, 0},  {ORDER_GROUPED, 16, 0}, {ORDER_GROUPED, 2, 1},
                                  {ORDER_GROUPED, 32, 1}, {ORDER_GROUPED, 2, 0},  {ORDER_GROUPED, 32, 0}};
    int64_t best_cost = -1, best_tiles = 0;
    SchedArgs best = *s;
    for (const Cand& c : kCands) {
        if (c.order == ORDER_GROUPED && c.G > s->nm) continue;   // the same map as a smaller G
        SchedArgs t = *s;
        t.order = c.order;
        t.group_m = c.G;
        t.remap = c.remap;
        int64_t cost, tiles;
        locality_cost(t, concurrent, &cost, &tiles);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_tiles = tiles;
            best = t;
        }
    }
    *s = best;
    *reuse_pm = best_tiles > 0 ? (int)(1000 - (1000 * best_cost) / (2 * best_tiles)) : 0;
}

// The compiler's resource report of a kernel, found through the symbol name of its
// launch handle (the handle's symbol carries the kernel's mangled name).
const KernelResources* resources_of(const void* fn) {
    Dl_info info;
    if (!fn || !dladdr(fn, &info) || !info.dli_sname) return nullptr;
    int lo = 0, hi = kNumKernelResources - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) / 2;
        const int c = strcmp(kKernelResources[mid].name, info.dli_sname);
        if (c == 0) return &kKernelResources[mid];
        if (c < 0) lo = mid + 1; else hi = mid - 1;
    }
    return nullptr;
}

// Shape-only checks and choices, shared by every entry point.  Row strides and
// base addresses (which only ts_gemm has) refine the vector flags later.
ts_status plan_shape(int64_t M, int64_t N, int64_t K, int32_t ab, int32_t c, const ts_schedule* sp,
                     Plan* p) {
    if (M < 0 || N < 0 || K < 0) return TS_ERR_INVALID_ARG;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return TS_ERR_UNSUPPORTED;
    if (ab == TS_F16 && c == TS_F16) p->io = IO_F16_F16;
    else if (ab == TS_F16 && c == TS_F32) p->io = IO_F16_F32;
    else if (ab == TS_BF16 && c == TS_BF16) p->io = IO_BF16_BF16;
    else if (ab == TS_BF16 && c == TS_F32) p->io = IO_BF16_F32;
    else if ((ab == TS_F16 || ab == TS_BF16 || ab == TS_F32) && (c == TS_F16 || c == TS_BF16 || c == TS_F32))
        return TS_ERR_UNSUPPORTED;
    else
        return TS_ERR_INVALID_ARG;

    ts_schedule s = {TS_ORDER_ROW_MAJOR, 1, TS_MODE_TILED, 0, 0, TS_TILE_AUTO, TS_INDEX_DIVIDE};
    if (sp) s = *sp;
    if (s.order != TS_ORDER_ROW_MAJOR && s.order != TS_ORDER_GROUPED && s.order != TS_ORDER_AUTO)
        return TS_ERR_INVALID_ARG;
    if (s.order == TS_ORDER_GROUPED && s.group_m < 1) return TS_ERR_INVALID_ARG;
    if (s.mode != TS_MODE_TILED && s.mode != TS_MODE_PERSISTENT && s.mode != TS_MODE_CROSSTILE &&
        s.mode != TS_MODE_STREAMK && s.mode != TS_MODE_AUTO)
        return TS_ERR_INVALID_ARG;
    if (s.index_math != TS_INDEX_DIVIDE && s.index_math != TS_INDEX_MULSHIFT) return TS_ERR_INVALID_ARG;
    if (s.num_programs < 0) return TS_ERR_INVALID_ARG;
    if (s.xcd_remap != 0 && s.xcd_remap != 1) return TS_ERR_INVALID_ARG;
    if (s.tile_config < TS_TILE_AUTO || s.tile_config > TS_TILE_256x256x64_PP) return TS_ERR_INVALID_ARG;

    int cfg = s.tile_config;
    if (cfg == TS_TILE_AUTO) {
        // largest tile that still gives the chip at least half a wave of tiles;
        // 256x256 tiles run with 8 waves (two per SIMD hide each other's stalls)
        if (cdiv64(M, 256) * cdiv64(N, 256) >= 128) cfg = CFG_256W8;
        else if (cdiv64(M, 128) * cdiv64(N, 128) >= 128) cfg = CFG_128;
        else cfg = CFG_64;
    }
    // the 4-wave 256 x 256 x 64 tile has no cross-tile kernel (see has_flat_kernel)
    if (cfg == CFG_256 && s.mode == TS_MODE_CROSSTILE) return TS_ERR_UNSUPPORTED;
    p->cfg = cfg;
    cfg_dims(cfg, &p->bm, &p->bn, &p->bk);
    const int64_t nm = cdiv64(M, p->bm), nn = cdiv64(N, p->bn), ks = cdiv64(K, p->bk);
    if (nm * nn > INT_MAX / 2 || ks > INT_MAX / 2) return TS_ERR_UNSUPPORTED;
    // the merged loop pays where tiles are short (small K), and wherever the nested
    // cross-tile kernel runs (at 16384^2 x 4096 it beat the persistent loop in 9 of
    // 9 interleaved rounds, by about 1 %)
    if (s.mode == TS_MODE_AUTO)
        s.mode = ((ks <= kCrossTileMaxSteps && cfg != CFG_256) || xtile_shape(cfg, ks)) ? TS_MODE_CROSSTILE
                                                                                          : TS_MODE_PERSISTENT;
    p->mode = s.mode;
    p->requested_programs = s.num_programs;
    p->s.nm = (int)nm;
    p->s.nn = (int)nn;
    p->s.ks = (int)ks;
    p->s.num_tiles = (int)(nm * nn);
    p->auto_order = s.order == TS_ORDER_AUTO;
    p->l2_reuse_pm = -1;
    p->s.order = p->auto_order ? TS_ORDER_ROW_MAJOR : s.order;
    p->s.group_m = s.order == TS_ORDER_GROUPED ? (int)(s.group_m < nm ? s.group_m : (nm > 0 ? nm : 1)) : 1;
    p->s.remap = p->auto_order ? 0 : s.xcd_remap;
    p->s.xcds = 8;
    p->s.grid = 0;
    p->s.fastdiv = s.index_math == TS_INDEX_MULSHIFT;
    // dense, 16-byte aligned operands assumed until ts_gemm sees the real ones
    const int64_t c_elem = c == TS_F32 ? 4 : 2;
    p->vec_a = (K % 8) == 0 ? 2 : (K % 2) == 0 ? 1 : 0;
    p->vec_b = (N % 8) == 0 ? 2 : (N % 2) == 0 ? 1 : 0;
    p->vec_c = (N * c_elem) % 16 == 0 ? 2 : (N * c_elem) % 8 == 0 ? 1 : 0;
    p->masked = (M % p->bm) != 0 || (N % p->bn) != 0 || (K % p->bk) != 0 || K == 0 ||
                p->vec_a != 2 || p->vec_b != 2 || p->vec_c != 2 ||
                (int64_t)p->bm * K * 2 > INT_MAX || (int64_t)p->bk * N * 2 > INT_MAX;
    p->path = choose_path(*p, N, K, 0, 0, K, N);
    return TS_OK;
}

// Workgroups one CU holds for the plan's kernel (needs a device).
int programs_per_cu(const Plan& p) {
    const KernelRef k = kernel_of(p);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k.fn, k.threads, 0) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    return n;
}

// Resolve the grid; cu/ppc of 0 mean "unknown" (host-only callers must pass
// num_programs explicitly in persistent modes).
ts_status resolve_grid(Plan* p, int cu_count, int ppc, int xcds) {
    p->s.xcds = xcds > 0 ? xcds : 8;
    if (p->s.num_tiles == 0) {
        p->s.grid = 0;
        p->max_items = 0;
        return TS_OK;
    }
    const int64_t ksp = p->s.ks > 0 ? p->s.ks : 1;
    if (p->mode == TS_MODE_TILED) {
        p->s.grid = p->s.num_tiles;
    } else {
        int64_t P = p->requested_programs;
        if (P == 0) {
            if (cu_count <= 0 || ppc <= 0) return TS_ERR_NO_DEVICE;
            P = (int64_t)cu_count * ppc;
        }
        // persistent: at most one program per tile; stream-K: per (tile, K step) item
        const int64_t cap = p->mode == TS_MODE_STREAMK ? (int64_t)p->s.num_tiles * ksp : p->s.num_tiles;
        p->s.grid = (int)(P < cap ? P : cap);
    }
    if (p->mode == TS_MODE_STREAMK) {
        const StreamK sk(p->s);
        p->max_items = cdiv64(sk.dp_tiles, p->s.grid) * ksp + sk.q + (sk.rem > 0 ? 1 : 0);
    } else {
        p->max_items = cdiv64(p->s.num_tiles, p->s.grid) * ksp;
    }
    // workgroups resident together: the device's CUs x workgroups per CU (256 CUs
    // and the plan's own grid when no device is known)
    const int64_t resident = (cu_count > 0 && ppc > 0) ? (int64_t)cu_count * ppc : 256;
    const int concurrent = (int)(resident < p->s.grid ? resident : p->s.grid);
    if (p->auto_order) {
        choose_order(&p->s, concurrent, &p->l2_reuse_pm);
    } else {
        int64_t cost, tiles;
        locality_cost(p->s, concurrent, &cost, &tiles);
        p->l2_reuse_pm = tiles > 0 ? (int)(1000 - (1000 * cost) / (2 * tiles)) : 0;
    }
    if (p->s.fastdiv) set_fastdiv(p->s);
    return TS_OK;
}

// Stream-K workspace of a resolved plan: a header of one flag per range plus an
// error counter (rounded up to 256 bytes), then one fp32 partial tile per range.
// Zero when the launch splits no tile.
struct WorkspaceLayout {
    int64_t header, part_bytes, total;
};
WorkspaceLayout workspace_layout(const Plan& p) {
    WorkspaceLayout w{0, 0, 0};
    if (p.mode != TS_MODE_STREAMK || p.s.grid == 0 || StreamK(p.s).sk_items == 0) return w;
    w.header = ((int64_t)(p.s.grid + 1) * 4 + 255) / 256 * 256;
    w.part_bytes = (int64_t)p.bm * p.bn * 4;
    w.total = w.header + (int64_t)p.s.grid * w.part_bytes;
    return w;
}

}  // namespace
}  // namespace ts

using namespace ts;

extern "C" const char* ts_status_string(ts_status status) {
    switch (status) {
        case TS_OK: return "TS_OK";
        case TS_ERR_INVALID_ARG: return "TS_ERR_INVALID_ARG: invalid argument";
        case TS_ERR_UNSUPPORTED: return "TS_ERR_UNSUPPORTED: unsupported dtype pair, stride pattern or size";
        case TS_ERR_ALIGNMENT: return "TS_ERR_ALIGNMENT: pointer not aligned to its element size";
        case TS_ERR_HIP: return "TS_ERR_HIP: HIP runtime error";
        case TS_ERR_NO_DEVICE: return "TS_ERR_NO_DEVICE: no usable GPU";
    }
    return "unknown ts_status";
}

// Sleeps (s_sleep 2, about 128 clocks each) before a stream-K wait gives up:
// about 2^24 * 128 clocks, roughly a second at the clocks the GEMM runs.
constexpr int kStreamKSpin = 1 << 24;

// use_scratch: the workspace is this library's per-device scratch array (the
// caller passes none); a launch that needs more than kScratchBytes is refused.
static ts_status gemm_launch(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                             int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                             int64_t stride_cm, int64_t stride_cn, int32_t ab_dtype, int32_t c_dtype,
                             const ts_schedule* sched, void* stream, uint64_t* clock_out, int64_t clock_rows,
                             void* workspace, int64_t workspace_bytes, bool use_scratch = false) {
    Plan p;
    ts_status st = plan_shape(M, N, K, ab_dtype, c_dtype, sched, &p);
    if (st != TS_OK) return st;
    if (M == 0 || N == 0) return TS_OK;
    if (!C || (K > 0 && (!A || !B))) return TS_ERR_INVALID_ARG;
    // Operand layouts: A stored [M][K] (stride_ak == 1) or [K][M] (stride_am == 1);
    // B stored [K][N] (stride_bn == 1) or [N][K] (stride_bk == 1); C stored [M][N].
    // A dimension of extent 1 makes its stride irrelevant: it is read as unit.
    if (M <= 1) stride_am = stride_ak == 1 ? stride_am : 1;
    if (K <= 1) { stride_ak = 1; stride_bk = stride_bn == 1 ? (stride_bk > N ? stride_bk : N) : 1; }
    if (N <= 1) stride_bn = stride_bk == 1 ? stride_bn : 1;
    if (stride_am < 0 || stride_ak < 0 || stride_bk < 0 || stride_bn < 0 || stride_cm < 0) return TS_ERR_INVALID_ARG;
    if (stride_cn != 1) return TS_ERR_UNSUPPORTED;
    const bool a_kmaj = stride_ak == 1, b_nmaj = stride_bn == 1;
    if (!(a_kmaj || stride_am == 1) || !(b_nmaj || stride_bk == 1)) return TS_ERR_UNSUPPORTED;
    const int64_t lda = a_kmaj ? stride_am : stride_ak;    // distance between stored rows
    const int64_t ldb = b_nmaj ? stride_bk : stride_bn;
    if ((a_kmaj && M > 1 && K > 0 && lda < K) || (!a_kmaj && K > 1 && lda < M) ||
        (b_nmaj && K > 1 && ldb < N) || (!b_nmaj && N > 1 && K > 0 && ldb < K) || (M > 1 && stride_cm < N))
        return TS_ERR_INVALID_ARG;
    if (lda > INT_MAX || ldb > INT_MAX || stride_cm > INT_MAX) return TS_ERR_UNSUPPORTED;
    const uintptr_t a = (uintptr_t)A, b = (uintptr_t)B, c = (uintptr_t)C;
    const int c_elem = c_dtype == TS_F32 ? 4 : 2;
    if ((a & 1) || (b & 1) || (c % c_elem)) return TS_ERR_ALIGNMENT;

    // Alignment levels of the rows: 16-byte operand vectors need 16-byte aligned
    // rows, 4-byte pieces 4-byte aligned ones; C vectors are 4 elements, pieces 2.
    // A stored [K][M] is gathered element by element (level 0 for its vectors).
    // A stored [K][M] is either staged whole by the direct-to-LDS loads (16-byte
    // aligned rows) or gathered element by element (level 0 for its vectors).
    p.vec_a = !a_kmaj ? ((a % 16 == 0) && (lda % 8 == 0) ? 2 : 0)
              : (a % 16 == 0) && (lda % 8 == 0 || M == 1) ? 2
              : (a % 4 == 0) && (lda % 2 == 0 || M == 1) ? 1 : 0;
    p.vec_b = (b % 16 == 0) && (ldb % 8 == 0 || (b_nmaj ? K <= 1 : N <= 1)) ? 2
              : (b % 4 == 0) && (ldb % 2 == 0 || (b_nmaj ? K <= 1 : N <= 1)) ? 1 : 0;
    p.vec_c = (c % (4 * c_elem) == 0) && (stride_cm % 4 == 0 || M == 1) ? 2
              : (c % (2 * c_elem) == 0) && (stride_cm % 2 == 0 || M == 1) ? 1 : 0;
    p.masked = (M % p.bm) != 0 || (N % p.bn) != 0 || (K % p.bk) != 0 || K == 0 || p.vec_a != 2 ||
               p.vec_b != 2 || p.vec_c != 2;
    // The unmasked kernels form row offsets inside a tile as 32-bit byte counts; the
    // masked ones use full-width pointers.
    if ((int64_t)(a_kmaj ? p.bm : p.bk) * lda * 2 > INT_MAX || (int64_t)(b_nmaj ? p.bk : p.bn) * ldb * 2 > INT_MAX)
        p.masked = 1;
    if (a_kmaj && b_nmaj) {
        p.path = choose_path(p, N, K, a, b, lda, ldb);
    } else if (a_kmaj && !p.masked && cfg_has_fast_path(p.cfg)) {
        p.path = PATH_FULL_BT;   // whole tiles, B stored [N][K] (its rows 16-byte aligned)
    } else if (!a_kmaj && !p.masked && cfg_has_at_path(p.cfg)) {
        // whole tiles, A stored [K][M] (its rows 16-byte aligned), B either way
        p.path = b_nmaj ? PATH_FULL_AT : PATH_FULL_ATBT;
    } else {
        p.path = PATH_MASKED;    // ragged or unaligned with a transposed operand; the 64x64x32 tile
        p.masked = true;
    }

    auto workspace_check = [&](const Plan& q) -> ts_status {
        const WorkspaceLayout w = workspace_layout(q);
        if (use_scratch) return w.total <= kScratchBytes ? TS_OK : TS_ERR_UNSUPPORTED;
        return (w.total == 0 || (workspace && workspace_bytes >= w.total && ((uintptr_t)workspace % 256) == 0))
                   ? TS_OK : TS_ERR_INVALID_ARG;
    };
    const bool grid_needs_device = p.mode != TS_MODE_TILED && p.requested_programs == 0;
    if (!grid_needs_device) {   // the workspace check needs no device here: report it first
        Plan q = p;
        st = resolve_grid(&q, 0, 0, 8);
        if (st != TS_OK) return st;
        st = workspace_check(q);
        if (st != TS_OK) return st;
    }
    int dev;
    DeviceInfo di;
    st = current_device(&dev, &di);
    if (st != TS_OK) return st;
    const int ppc = (grid_needs_device || p.auto_order) ? programs_per_cu(p) : 1;
    st = resolve_grid(&p, di.cu_count, ppc, di.xcds);
    if (st != TS_OK) return st;
    if (clock_out && clock_rows < p.s.grid) return TS_ERR_INVALID_ARG;
    st = workspace_check(p);
    if (st != TS_OK) return st;
    const WorkspaceLayout wl = workspace_layout(p);
    if (use_scratch && wl.total > 0) {
        st = scratch_ptr(dev, &workspace);
        if (st != TS_OK) return st;
        // the array keeps the last call's contents: clear the flags and the timeout
        // counter (a fill kernel, so that the call can be captured in a graph)
        const int words = (int)(wl.header / 4);
        hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                           static_cast<int*>(workspace), words);
        if (hipGetLastError() != hipSuccess) return TS_ERR_HIP;
    }

    GemmArgs g;
    g.A = static_cast<const uint16_t*>(A);
    g.B = static_cast<const uint16_t*>(B);
    g.C = C;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = stride_cm;
    g.sam = stride_am;
    g.sak = stride_ak;
    g.sbk = stride_bk;
    g.sbn = stride_bn;
    g.vec_a = p.vec_a;
    g.vec_b = p.vec_b;
    g.vec_c = p.vec_c;
    {
        const int64_t pitch = stride_cm * c_elem;
        int ca = 16;
        while (ca > 2 && ((c % ca) != 0 || (M > 1 && pitch % ca != 0))) ca >>= 1;
        g.c_align = ca;
    }
    g.a_bytes = K > 0 ? ((M - 1) * stride_am + (K - 1) * stride_ak + 1) * 2 : 0;
    g.b_bytes = K > 0 ? ((K - 1) * stride_bk + (N - 1) * stride_bn + 1) * 2 : 0;
    g.s = p.s;
    g.clk = reinterpret_cast<unsigned long long*>(clock_out);
    g.sk_flags = wl.total > 0 ? static_cast<int*>(workspace) : nullptr;
    g.sk_err = wl.total > 0 ? static_cast<int*>(workspace) + p.s.grid : nullptr;
    g.sk_part = wl.total > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.header) : nullptr;
    g.sk_spin = kStreamKSpin;
    const KernelRef k = kernel_of(p);
    void* args[] = {&g};
    if (hipLaunchKernel(k.fn, dim3(p.s.grid), dim3(k.threads), args, 0, (hipStream_t)stream) != hipSuccess) {
        (void)hipGetLastError();
        return TS_ERR_HIP;
    }
    return TS_OK;
}

extern "C" ts_status ts_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                             int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                             int64_t stride_cm, int64_t stride_cn, int32_t ab_dtype, int32_t c_dtype,
                             const ts_schedule* sched, void* stream) {
    return gemm_launch(A, B, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       ab_dtype, c_dtype, sched, stream, nullptr, 0, nullptr, 0);
}

extern "C" ts_status ts_gemm_workspace(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                       int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                                       int64_t stride_cm, int64_t stride_cn, int32_t ab_dtype, int32_t c_dtype,
                                       const ts_schedule* sched, void* stream, void* workspace,
                                       int64_t workspace_bytes) {
    if (workspace_bytes < 0) return TS_ERR_INVALID_ARG;
    return gemm_launch(A, B, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       ab_dtype, c_dtype, sched, stream, nullptr, 0, workspace, workspace_bytes);
}

extern "C" ts_status ts_gemm_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                     int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                                     int64_t stride_cm, int64_t stride_cn, int32_t ab_dtype, int32_t c_dtype,
                                     const ts_schedule* sched, void* stream) {
    return gemm_launch(A, B, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       ab_dtype, c_dtype, sched, stream, nullptr, 0, nullptr, 0, true);
}

extern "C" int64_t ts_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" ts_status ts_gemm_clocked(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                     int64_t stride_am, int64_t stride_ak, int64_t stride_bk, int64_t stride_bn,
                                     int64_t stride_cm, int64_t stride_cn, int32_t ab_dtype, int32_t c_dtype,
                                     const ts_schedule* sched, void* stream, uint64_t* clock_out,
                                     int64_t clock_rows, void* workspace, int64_t workspace_bytes) {
    if (!clock_out || workspace_bytes < 0) return TS_ERR_INVALID_ARG;
    return gemm_launch(A, B, C, M, N, K, stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn,
                       ab_dtype, c_dtype, sched, stream, clock_out, clock_rows, workspace, workspace_bytes);
}

extern "C" ts_status ts_query(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                              const ts_schedule* sched, ts_launch_info* out) {
    if (!out) return TS_ERR_INVALID_ARG;
    Plan p;
    ts_status st = plan_shape(M, N, K, ab_dtype, c_dtype, sched, &p);
    if (st != TS_OK) return st;
    int dev;
    DeviceInfo di;
    const bool have_dev = current_device(&dev, &di) == TS_OK;
    const int ppc = have_dev ? programs_per_cu(p) : 0;
    st = resolve_grid(&p, have_dev ? di.cu_count : 0, ppc, have_dev ? di.xcds : 8);
    if (st != TS_OK) return st;
    const KernelRef k = kernel_of(p);
    out->block_m = p.bm;
    out->block_n = p.bn;
    out->block_k = p.bk;
    out->threads = k.threads;
    out->num_m_tiles = p.s.nm;
    out->num_n_tiles = p.s.nn;
    out->k_steps = p.s.ks;
    out->num_tiles = p.s.num_tiles;
    out->grid = p.s.grid;
    out->programs_per_cu = ppc;
    out->cu_count = have_dev ? di.cu_count : 0;
    out->xcds = p.s.xcds;
    out->lds_bytes = k.lds_bytes;
    out->masked = p.path;
    out->workspace_bytes = workspace_layout(p).total;
    out->trace_items = p.max_items;
    out->order = p.s.order;
    out->group_m = p.s.group_m;
    out->mode = p.mode;
    out->xcd_remap = p.s.remap;
    out->index_math = p.s.fastdiv ? TS_INDEX_MULSHIFT : TS_INDEX_DIVIDE;
    out->model_l2_reuse_pm = p.l2_reuse_pm;
    out->vgprs = -1;
    out->scratch_bytes = -1;
    const KernelResources* kr = resources_of(k.fn);
    out->arch_vgprs = kr ? kr->vgprs : -1;
    out->agprs = kr ? kr->agprs : -1;
    out->sgprs = kr ? kr->sgprs : -1;
    out->spilled_vgprs = kr ? kr->vgpr_spill : -1;
    out->spilled_sgprs = kr ? kr->sgpr_spill : -1;
    out->compiler_occupancy = kr ? kr->occupancy : -1;
    if (have_dev) {
        hipFuncAttributes fa;
        if (hipFuncGetAttributes(&fa, k.fn) == hipSuccess) {
            out->vgprs = fa.numRegs;
            out->scratch_bytes = (int32_t)fa.localSizeBytes;
            out->lds_bytes = (int32_t)fa.sharedSizeBytes;
        } else {
            (void)hipGetLastError();
        }
    }
    return TS_OK;
}

extern "C" ts_status ts_schedule_trace_host(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                                            const ts_schedule* sched, int32_t cu_count, int32_t ppc,
                                            int32_t* out, int64_t out_rows) {
    Plan p;
    ts_status st = plan_shape(M, N, K, ab_dtype, c_dtype, sched, &p);
    if (st != TS_OK) return st;
    st = resolve_grid(&p, cu_count, ppc, 8);
    if (st != TS_OK) return st;
    const int64_t need = (int64_t)p.s.grid * p.max_items;
    if (need == 0) return TS_OK;
    if (!out || out_rows < need) return TS_ERR_INVALID_ARG;
    for (int prog = 0; prog < p.s.grid; ++prog)
        trace_program(p.s, p.mode, prog, (int)p.max_items, out + (int64_t)prog * p.max_items * 5);
    return TS_OK;
}

extern "C" ts_status ts_schedule_trace(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                                       const ts_schedule* sched, int32_t* out, int64_t out_rows, void* stream) {
    Plan p;
    ts_status st = plan_shape(M, N, K, ab_dtype, c_dtype, sched, &p);
    if (st != TS_OK) return st;
    int dev;
    DeviceInfo di;
    st = current_device(&dev, &di);
    if (st != TS_OK) return st;
    const int ppc = ((p.mode != TS_MODE_TILED && p.requested_programs == 0) || p.auto_order) ? programs_per_cu(p) : 1;
    st = resolve_grid(&p, di.cu_count, ppc, di.xcds);
    if (st != TS_OK) return st;
    const int64_t need = (int64_t)p.s.grid * p.max_items;
    if (need == 0) return TS_OK;
    if (!out || out_rows < need) return TS_ERR_INVALID_ARG;
    if (need * 5 > INT_MAX) return TS_ERR_UNSUPPORTED;
    const int threads = 256;
    hipLaunchKernelGGL(trace_kernel, dim3((p.s.grid + threads - 1) / threads), dim3(threads), 0,
                       (hipStream_t)stream, p.s, p.mode, (int)p.max_items, out);
    if (hipGetLastError() != hipSuccess) return TS_ERR_HIP;
    return TS_OK;
}
