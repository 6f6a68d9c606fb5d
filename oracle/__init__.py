"""CPU oracle for the tiled GEMM and its tile-order schedules.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, loads or calls
this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the GPU library.

Contents
  gemm      -- fp64 matrix product of fp16/bf16 inputs (C library ref_gemm.c,
               plus a pure-Python loop for tiny cases) and the acceptance bound
  schedule  -- the tile-order maps (row-major, grouped, XCD remap, persistent,
               flattened cross-tile) as plain Python integer functions
  model     -- the counting model of the roofline and tiling notes (FLOPs,
               element reads with and without reuse, bytes, intensity, roofline,
               on-chip bytes, panel sizes, block limits)

Every function cites the passage of the pages it follows.  Parity status of
each function is stated in its module header.
"""
