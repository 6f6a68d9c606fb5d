/*
 * tsgemm -- tiled dense matrix multiply with tile-order schedules, for AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (from "Week-4 notes: Roofline and Tiling", section 1, and the
 * naive tiled matmul listing of "(1/n) Triton matmul ... persistent kernel"):
 *
 *     C[M,N] = A[M,K] @ B[K,N]       C[i][j] = sum_k A[i][k] * B[k][j]
 *
 * with fp16 or bf16 inputs, an fp32 accumulator held on chip for the whole K
 * loop, and one conversion of the accumulator to the output type (round to
 * nearest even) when the output tile is stored.  The output C is split into
 * BLOCK_M x BLOCK_N tiles; the schedule decides which workgroup computes which
 * tile and in what order (see ts_schedule below).
 *
 * Conventions shared by every entry point
 *   - Matrix pointers are DEVICE pointers, owned by the caller; the library never
 *     frees them and keeps no reference after the call is enqueued.
 *   - Strides are in ELEMENTS, as in the pages' kernels: element (i,k) of A is
 *     A[i*stride_am + k*stride_ak], (k,j) of B is B[k*stride_bk + j*stride_bn],
 *     (i,j) of C is C[i*stride_cm + j*stride_cn].
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without synchronising.
 *   - Arguments are validated on the host before any HIP call; an invalid call
 *     returns an error code and enqueues nothing.  No entry point allocates
 *     device memory.
 *   - Thread-safe: the only state is a per-device cache of device properties.
 */
#ifndef TSGEMM_H
#define TSGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TS_OK = 0,
    TS_ERR_INVALID_ARG = -1,  /* null pointer with work to do, negative size, bad stride, bad schedule */
    TS_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement (dtype pair, stride pattern) */
    TS_ERR_ALIGNMENT = -3,    /* a pointer is not aligned to its element size */
    TS_ERR_HIP = -4,          /* the HIP runtime reported an error (query or launch) */
    TS_ERR_NO_DEVICE = -5     /* the request needs a GPU and none is usable */
} ts_status;

/* element types */
enum { TS_F16 = 1, TS_BF16 = 2, TS_F32 = 3 };

/* tile order: which output tile a linear tile id denotes */
enum {
    /* tile_m = id / num_n_tiles, tile_n = id % num_n_tiles
       ("(1/n) ... persistent kernel", naive tiled matmul listing) */
    TS_ORDER_ROW_MAJOR = 0,
    /* grouped ordering / CTA swizzle: ids walk GROUP_SIZE_M tile rows at a time,
       M coordinate first; the last group holds the remaining num_m_tiles mod G
       rows ("(2/n) ... grouped ordering (CTA swizzle)", section Implementation) */
    TS_ORDER_GROUPED = 1,
    /* chosen per shape by the library (group_m and xcd_remap are ignored): among
       row-major and grouped orders with G in {2, 4, 8, 16, 32}, each with and
       without the XCD remap, the one whose first round of workgroups touches the
       fewest distinct tile rows and tile columns per XCD (a model of L2 reuse:
       each XCD has its own L2); ties go to the earlier candidate in the order
       G=8+remap, G=4+remap, G=16+remap, row-major, row-major+remap, G=8, G=4,
       G=16, G=2+remap, G=32+remap, G=2, G=32.  The grouping page's closing
       section says the best order depends on the size and the cache; this is
       that choice made from a model rather than a sweep.  The model counts operand
       reuse only: at a few K steps per tile, where writing C is most of the traffic,
       the fastest order varies with C's row pitch and the number of tile rows, and
       an explicit order can be faster.  ts_query reports the resolved order, G and
       remap. */
    TS_ORDER_AUTO = 2
};

/* how workgroups take tiles */
enum {
    /* one workgroup per tile; the hardware dispatcher assigns them */
    TS_MODE_TILED = 0,
    /* P = min(num_programs, num_tiles) workgroups; workgroup p computes tile ids
       p, p+P, p+2P, ... ("(1/n) ...", naive persistent listing and grid code) */
    TS_MODE_PERSISTENT = 1,
    /* as PERSISTENT, but the tile loop and the K loop are one flattened loop, so
       the next tile's first K slices are fetched while the current tile is being
       stored ("(3/n) ... cross tile pipelining", merged loop).  On the 128x128x64
       and 8-wave 256x256x64 tiles, when the direct-to-LDS pipeline runs
       (ts_launch_info.masked 0, 2-5) and a tile has at least 2 K steps (with one
       tile per program: at least 8), the same (tile, k) sequence runs as a tile
       loop with the K loop inside and the next tile's first two slices loaded by
       the last two K steps. */
    TS_MODE_CROSSTILE = 2,
    /* stream-K, the follow-on the persistent page names for its tail (the split is
       this library's design): the first num_tiles - (num_tiles mod P) tiles run as
       in PERSISTENT; the (tile, K step) items of the remaining tiles are dealt to all
       P programs as contiguous ranges of equal length (+-1), program p taking range
       P-1-p.  The program holding K step 0 of a split tile adds the other ranges'
       fp32 partial tiles, in range order, and stores it; the result is identical
       from run to run but not bit-identical to the other modes (a different
       summation order along K).  Needs a workspace: ts_gemm_workspace, sized by
       ts_query's workspace_bytes (0 when no tile is split). */
    TS_MODE_STREAMK = 3,
    /* chosen by the library: TS_MODE_CROSSTILE when a tile has at most 32 K
       steps (the cross-tile page finds the merged loop paying where the tile
       boundary is a large share of the work, i.e. at small K), or at least 8 on
       the 128x128x64 and 8-wave 256x256x64 tiles (where the nested form above
       runs), else TS_MODE_PERSISTENT.  ts_query reports the
       resolved mode. */
    TS_MODE_AUTO = 4
};

/* index arithmetic of the tile-order maps */
enum {
    TS_INDEX_DIVIDE = 0,     /* integer division and remainder                            */
    TS_INDEX_MULSHIFT = 1    /* multiply-high and shift by multipliers made on the host
                                (Granlund and Montgomery 1994); the same map, bit for bit */
};

/* tile configurations (BLOCK_M x BLOCK_N x BLOCK_K) */
enum {
    TS_TILE_AUTO = 0,          /* library chooses from the shape */
    TS_TILE_64x64x32 = 1,
    TS_TILE_128x128x64 = 2,
    TS_TILE_256x256x64 = 3,    /* 4 waves of 128x128 (one per SIMD); tiled and persistent
                                  modes only (TS_MODE_CROSSTILE: TS_ERR_UNSUPPORTED) */
    TS_TILE_256x256x64_W8 = 4, /* 8 waves of 128x64 (two per SIMD)   */
    TS_TILE_256x256x64_PP = 5  /* the _W8 tile and wave layout run as two groups of four
                                  waves that take turns: in each phase of a K step one
                                  group multiplies while the other reads its next
                                  fragments from LDS.  Each program's tiles form one
                                  stream of (tile, K step) items, so the tile boundary
                                  does not drain the pipeline in any mode.  Stream-K and
                                  the masked register path run the _W8 kernels.       */
};

typedef struct {
    int32_t order;         /* TS_ORDER_*                                                      */
    int32_t group_m;       /* GROUP_SIZE_M >= 1, read when order == TS_ORDER_GROUPED; values
                              above num_m_tiles act as num_m_tiles (column-major order)       */
    int32_t mode;          /* TS_MODE_*                                                       */
    int32_t num_programs;  /* persistent modes: workgroups to launch; 0 = number of CUs times
                              the workgroups one CU holds for the chosen kernel; always capped
                              at num_tiles.  Ignored for TS_MODE_TILED.                        */
    int32_t xcd_remap;     /* 1 = renumber workgroups so that each XCD (chiplet with its own
                              L2) works on one contiguous run of tile ids; 0 = off             */
    int32_t tile_config;   /* TS_TILE_*                                                       */
    int32_t index_math;    /* TS_INDEX_*                                                      */
} ts_schedule;

typedef struct {
    int32_t block_m, block_n, block_k;  /* tile shape used                                   */
    int32_t threads;                    /* threads per workgroup                             */
    int64_t num_m_tiles, num_n_tiles;   /* cdiv(M, block_m), cdiv(N, block_n)                 */
    int64_t k_steps;                    /* cdiv(K, block_k)                                   */
    int64_t num_tiles;                  /* num_m_tiles * num_n_tiles                          */
    int64_t grid;                       /* workgroups launched                                */
    int32_t programs_per_cu;            /* workgroups one CU holds (0 if no device)           */
    int32_t cu_count;                   /* compute units of the current device (0 if none)    */
    int32_t xcds;                       /* XCDs the workgroups are dealt over (8 if no device) */
    int32_t lds_bytes;                  /* LDS per workgroup                                   */
    int32_t masked;                     /* kernel path: 0 whole tiles; 1 masked register        */
                                        /* pipeline (ragged or unaligned); 2 direct-to-LDS      */
                                        /* pipeline with edges zero-filled by the loads' range  */
                                        /* checks; 3 whole tiles with B stored [N][K]; 4 whole  */
                                        /* tiles with A stored [K][M]; 5 both.  ts_query        */
                                        /* assumes dense, 16-byte aligned A [M][K] and B [K][N];*/
                                        /* by ts_gemm's layout rules, a transposed operand      */
                                        /* takes path 3, 4 or 5 where this reports 0 (4 and 5   */
                                        /* on the square tiles, not 64x64x32), else path 1.     */
    int64_t workspace_bytes;            /* TS_MODE_STREAMK: workspace the launch needs (0: none) */
    int64_t trace_items;                /* most (tile, K step) items of one workgroup: the row
                                           stride of ts_schedule_trace's output                */
    int32_t vgprs;                      /* registers per thread reported by the runtime (-1 if none) */
    int32_t scratch_bytes;              /* private (spill) bytes per thread (-1 if none)       */
    /* The compiler's resource report for the kernel, recorded when the library was
       built (available without a device; -1 if the kernel is missing from it).   */
    int32_t arch_vgprs;                 /* architectural vector registers per lane             */
    int32_t agprs;                      /* accumulation registers (AGPRs) per lane             */
    int32_t sgprs;                      /* scalar registers per wave                           */
    int32_t spilled_vgprs;              /* vector registers spilled to private memory          */
    int32_t spilled_sgprs;              /* scalar registers spilled                            */
    int32_t compiler_occupancy;         /* waves per SIMD the compiler computed                */
    /* the schedule as resolved (TS_ORDER_AUTO / TS_MODE_AUTO replaced by the choice) */
    int32_t order, group_m, mode, xcd_remap, index_math;
    int32_t model_l2_reuse_pm;          /* the L2 model's reuse fraction of the resolved order,
                                           in 1/1000: 1 - distinct tile rows and columns per
                                           XCD over 2 x tiles, in the first round          */
} ts_launch_info;

/*
 * C = A @ B on `stream`.
 *   A: M x K, B: K x N, C: M x N, strides as above.  Supported layouts: A stored
 *   [M][K] (stride_ak == 1, stride_am >= K) or [K][M] (stride_am == 1,
 *   stride_ak >= M); B stored [K][N] (stride_bn == 1, stride_bk >= N) or [N][K]
 *   (stride_bk == 1, stride_bn >= K); C stored [M][N] (stride_cn == 1,
 *   stride_cm >= N).  A dimension of extent 1 makes its stride irrelevant.  Any
 *   other stride pattern returns TS_ERR_UNSUPPORTED; a row stride below its row's
 *   length, TS_ERR_INVALID_ARG.  Whole tiles with B stored [N][K] run the
 *   direct-to-LDS pipeline with B's slices staged as A's (kernel path 3); whole
 *   tiles with A stored [K][M] run it with A's slices staged as B's (paths 4 and 5;
 *   16-byte aligned rows).  Ragged shapes with a transposed operand run the masked
 *   register pipeline, which gathers it element by element.
 *   ab_dtype / c_dtype: TS_F16 -> TS_F16 or TS_F32; TS_BF16 -> TS_BF16 or TS_F32.
 *   M == 0 or N == 0: nothing to do, TS_OK.  K == 0: C is set to zero.
 *   Ragged M, N, K and row strides that defeat 16-byte vector access are handled
 *   by masked loads and stores (out-of-range A and B elements read as zero; C is
 *   written only inside M x N).  When K and A's row stride are multiples of 8
 *   elements with A 16-byte aligned, and B's base is 4-byte aligned with its row
 *   stride and N even, the edges are zero-filled by the direct-to-LDS loads themselves
 *   (no element-wise masking).  sched == NULL means row-major tiled, auto tile.
 *   The result does not depend on the schedule: every schedule with the same tile
 *   configuration produces bit-identical C.
 *   Errors: TS_ERR_INVALID_ARG / TS_ERR_UNSUPPORTED / TS_ERR_ALIGNMENT before any
 *   HIP call; TS_ERR_NO_DEVICE if no GPU; TS_ERR_HIP if the launch fails.
 *   A TS_MODE_STREAMK launch that splits tiles needs a workspace: call
 *   ts_gemm_workspace (here it returns TS_ERR_INVALID_ARG).
 */
ts_status ts_gemm(const void* A, const void* B, void* C,
                  int64_t M, int64_t N, int64_t K,
                  int64_t stride_am, int64_t stride_ak,
                  int64_t stride_bk, int64_t stride_bn,
                  int64_t stride_cm, int64_t stride_cn,
                  int32_t ab_dtype, int32_t c_dtype,
                  const ts_schedule* sched, void* stream);

/*
 * ts_gemm with a caller-owned device workspace, for schedules that need one
 * (TS_MODE_STREAMK; see there).  workspace_bytes must be at least ts_query's
 * workspace_bytes for the same arguments and the workspace 256-byte aligned,
 * else TS_ERR_INVALID_ARG; launches that need no workspace accept NULL.
 * Layout: int32 flags[P] (P = ts_query's grid), int32 timeouts, padding to 256
 * bytes, then P partial tiles of block_m x block_n fp32.  The header (flags and
 * timeout counter) must be zero before the first call on a workspace; every
 * call leaves the flags zero again.  The timeout counter counts waits for
 * another workgroup's partial tile that gave up after about a second (possible
 * only if other work keeps that workgroup from running; the result is then
 * wrong); it is never reset by the library.  Calls that share a workspace must
 * not overlap in time (use one stream, or one workspace per stream).
 * Otherwise as ts_gemm.
 */
ts_status ts_gemm_workspace(const void* A, const void* B, void* C,
                            int64_t M, int64_t N, int64_t K,
                            int64_t stride_am, int64_t stride_ak,
                            int64_t stride_bk, int64_t stride_bn,
                            int64_t stride_cm, int64_t stride_cn,
                            int32_t ab_dtype, int32_t c_dtype,
                            const ts_schedule* sched, void* stream,
                            void* workspace, int64_t workspace_bytes);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ts_gemm_workspace without
 * a workspace argument.  A launch that needs a workspace (TS_MODE_STREAMK with
 * split tiles) uses this library's own scratch array instead, a static device
 * array of ts_noalloc_scratch_bytes() bytes (64 MiB + 64 KiB) of which every GPU
 * the library runs on holds one copy until the process ends; a launch that would
 * need more returns TS_ERR_UNSUPPORTED before any HIP call (query workspace_bytes
 * first).  The call allocates nothing: before the GEMM it enqueues one small
 * kernel that clears the scratch array's flags.  Every call on a GPU shares that
 * GPU's array, so calls that overlap in time on one GPU (on different streams,
 * or from different threads) race and must not be made.  Otherwise as
 * ts_gemm_workspace; launches that need no workspace behave exactly as ts_gemm.
 */
ts_status ts_gemm_noalloc(const void* A, const void* B, void* C,
                          int64_t M, int64_t N, int64_t K,
                          int64_t stride_am, int64_t stride_ak,
                          int64_t stride_bk, int64_t stride_bn,
                          int64_t stride_cm, int64_t stride_cn,
                          int32_t ab_dtype, int32_t c_dtype,
                          const ts_schedule* sched, void* stream);

/* Size in bytes of the scratch array ts_gemm_noalloc uses (the largest workspace
   it accepts). */
int64_t ts_noalloc_scratch_bytes(void);

/*
 * This library's own addition, for measurement: ts_gemm with a clock record: the same product, launch and
 * errors, and in addition thread 0 of every workgroup p writes four counters to
 * the device buffer clock_out (owned by the caller, clock_rows x 4 uint64):
 *   clock_out[4p + 0 .. 1] = shader-clock counter (s_memtime) at the start and end
 *                            of the workgroup,
 *   clock_out[4p + 2 .. 3] = constant 100 MHz counter (s_memrealtime) at the same
 *                            two points,
 * so (end - start) of the first over (end - start) of the second, times 100 MHz,
 * is the shader clock the workgroup ran at.  Used to state a kernel's MFMA
 * utilisation at the clock the board's power limit actually allowed.
 * clock_rows must be >= the launch grid (ts_query), else TS_ERR_INVALID_ARG;
 * clock_out == NULL is TS_ERR_INVALID_ARG.  workspace / workspace_bytes: as in
 * ts_gemm_workspace (NULL / 0 when the schedule needs none).
 */
ts_status ts_gemm_clocked(const void* A, const void* B, void* C,
                          int64_t M, int64_t N, int64_t K,
                          int64_t stride_am, int64_t stride_ak,
                          int64_t stride_bk, int64_t stride_bn,
                          int64_t stride_cm, int64_t stride_cn,
                          int32_t ab_dtype, int32_t c_dtype,
                          const ts_schedule* sched, void* stream,
                          uint64_t* clock_out, int64_t clock_rows,
                          void* workspace, int64_t workspace_bytes);

/*
 * This library's own addition, a measurement probe: one workgroup of 8 waves per compute unit, each wave running
 * `iters` rounds of 8 independent v_mfma_f32_32x32x16_f16 with no memory traffic,
 * enqueued on `stream`.  Its operands are constants held in registers, whose low
 * toggle rate draws less power than a GEMM on random data, so its rate is an upper
 * bound on what the matrix cores sustain, not the rate at a GEMM's power draw.  Times the matrix cores' sustained rate on this device
 * when the caller brackets it with events: *flops (host pointer) receives the
 * floating-point operations the launch executes.  `sink` is a caller-owned device
 * buffer of at least (compute units x 512) floats that receives one value per
 * thread (the accumulators' sum, so that no MFMA is dead code).
 * Errors: TS_ERR_INVALID_ARG (iters <= 0, null pointers, sink too small),
 * TS_ERR_NO_DEVICE, TS_ERR_HIP (launch failure).
 */
ts_status ts_mfma_loop_probe(int32_t iters, float* sink, int64_t sink_elems, double* flops, void* stream);

/* ts_mfma_phase_probe: the probe above with its MFMA stream cut by workgroup barriers,
 * the cost of a barrier pattern on its own (no memory traffic).  This library's own
 * measurement addition, for the choice between one barrier per K half-step and the
 * ping-pong kernel's alternating phases.  Per iteration every wave issues 16 MFMAs
 * (pattern 3: 32):
 *   0  no barrier;
 *   1  every wave: 8 MFMAs, barrier, 8 MFMAs, barrier;
 *   2  ping-pong: waves 0-3 issue 16 MFMAs while waves 4-7 wait at a barrier, then the
 *      other way round;
 *   3  ping-pong with 32-MFMA phases.
 * Operands are the same constants as the loop probe's.  `sink` as there; `flops`
 * receives the launch's FLOPs.  Errors: TS_ERR_INVALID_ARG (iters <= 0, pattern
 * outside 0..3, null or short sink, null flops), TS_ERR_NO_DEVICE, TS_ERR_HIP.
 * Asynchronous on `stream`. */
ts_status ts_mfma_phase_probe(int32_t iters, int32_t pattern, float* sink, int64_t sink_elems, double* flops,
                              void* stream);

/*
 * This library's own addition (the pages print no such trace): writes the work
 * sequence of every workgroup, computed on the GPU by the same
 * device functions the GEMM kernels use, to the device buffer `out` of
 * out_rows x 5 int32: row (p * max_items + it) = (p, it, tile_m, tile_n, k_step)
 * for the it-th (tile, K-step) item workgroup p processes, where max_items =
 * ts_query's trace_items (cdiv(num_tiles, grid) * max(k_steps, 1) except in
 * stream-K mode); rows past a workgroup's item count are filled with -1.
 * out_rows must be >= grid * max_items.
 * Same validation and error codes as ts_gemm (no matrix pointers involved).
 */
ts_status ts_schedule_trace(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                            const ts_schedule* sched, int32_t* out, int64_t out_rows, void* stream);

/*
 * This library's own addition: host-side twin of ts_schedule_trace: the same schedule functions run on the
 * CPU into the host buffer `out`.  `cu_count` and `programs_per_cu` stand in for
 * the device when sched->num_programs == 0 in a persistent mode.  No HIP call.
 */
ts_status ts_schedule_trace_host(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                                 const ts_schedule* sched, int32_t cu_count, int32_t programs_per_cu,
                                 int32_t* out, int64_t out_rows);

/*
 * Fills `out` with the launch ts_gemm would make for these arguments (tile
 * shape, tile counts, grid, occupancy, registers).
 *
 * The persistent grid follows the grid code of the naive persistent matmul in
 * "(1/n) Triton matmul ... persistent kernel" (num_programs = min(SMs x
 * programs_per_sm, num_tiles)), with CUs for SMs and, for programs_per_sm, the
 * workgroups one CU holds for the chosen kernel.  That page's section on
 * computing the block limit by hand derives programs_per_sm from the compiled
 * kernel's registers, spills and shared memory per block; here the HIP runtime's
 * occupancy calculation does it (programs_per_cu), and the kernel's resource use
 * is reported beside it: the runtime's register and private-memory figures
 * (vgprs, scratch_bytes, lds_bytes; device needed) and the compiler's own report
 * (arch_vgprs, agprs, sgprs, spills, compiler_occupancy; recorded at build time).
 *
 * Needs a device only when the grid depends on it (persistent mode with
 * num_programs == 0) or for the runtime's occupancy and register fields, which
 * are 0 / -1 without one.  Errors: as ts_gemm's argument checks.
 */
ts_status ts_query(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                   const ts_schedule* sched, ts_launch_info* out);

/* Static, human-readable name of a status code.  This library's own addition
   (the pages define no error reporting). */
const char* ts_status_string(ts_status status);

#ifdef __cplusplus
}
#endif

#endif /* TSGEMM_H */
