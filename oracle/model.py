"""Counting model of tiled GEMM traffic -- TEST INFRASTRUCTURE ONLY.

Follows "Week-4 notes: Roofline and Tiling":
  * section 1 (arithmetic intensity): I = FLOPs / bytes moved to and from HBM;
    a matrix product does 2MNK FLOPs;
  * section 2 (roofline): attainable = min(P, BW * I), ridge point = P / BW;
  * section 5.1 (the 4x4 example with 2x2 tiles): element reads with no reuse,
    with tiling and with everything on chip;
  * section 5.2 (general tile formulas): per step 2*BM*BN*BK FLOPs and
    BM*BK + BK*BN reads, per tile K*(BM + BN) reads, in total MNK(1/BM + 1/BN)
    reads and MN writes;
  * section 5.3 (4096^3 fp32 on P = 20 TFLOP/s, BW = 1 TB/s): ideal time =
    max(compute time, memory time);
  * section 5.4 (on-chip bytes): input slices plus the accumulator tile.
and "(2/n) ... grouped ordering", section "Reuse distance and cache capacity":
A panel = BLOCK_M * K * e bytes, B panel = K * BLOCK_N * e bytes; a row-major
tile row touches all B panels plus one A panel, a group of G tile rows touches
G A panels plus one B panel; and "(1/n) ... persistent kernel", sections
"Computing block limits" and "Grid size": a resource limit admits
floor(available / per-block) blocks, waves = grid / (SMs * blocks per SM).

For ragged shapes the tiled read count keeps only in-bounds elements (masked
loads fetch nothing): sum over tiles of K * (rows + cols) = K * (nn*M + nm*N).

The per-XCD L2 locality model at the end of this file is this library's own
(not on the pages): the pages' reuse-distance argument ("(2/n) ...", section
"Reuse distance and cache capacity") moved to a GPU whose XCDs each have their
own L2.  It is pinned by hand-worked cases and by the reuse fractions computed
for the tile grids of the 16384 x 16384 product when the build was planned.

Parity pins: every number the notes and pages print for these quantities
(tests/test_oracle_model.py).
"""
from __future__ import annotations

import math


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def flops_step(BM: int, BN: int, BK: int) -> int:
    return 2 * BM * BN * BK


def reads_no_reuse(M: int, N: int, K: int) -> int:
    """Every output reads its own row of A and column of B: MN * (K + K) elements."""
    return M * N * 2 * K


def reads_step(BM: int, BN: int, BK: int) -> int:
    return BM * BK + BK * BN


def reads_tile(BM: int, BN: int, K: int) -> int:
    return K * (BM + BN)


def reads_tiled(M: int, N: int, K: int, BM: int, BN: int) -> int:
    """Sum over output tiles of the in-bounds A and B elements each one loads."""
    nm, nn = cdiv(M, BM), cdiv(N, BN)
    total = 0
    for tm in range(nm):
        rows = min(BM, M - tm * BM)
        for tn in range(nn):
            cols = min(BN, N - tn * BN)
            total += K * (rows + cols)
    return total


def reads_ideal(M: int, N: int, K: int) -> int:
    return M * K + K * N


def writes(M: int, N: int) -> int:
    return M * N


def traffic_bytes(reads: int, wr: int, elem: int) -> int:
    return elem * (reads + wr)


def intensity(fl: float, nbytes: float) -> float:
    return fl / nbytes


def roofline(P: float, BW: float, I: float) -> float:
    return min(P, BW * I)


def ridge(P: float, BW: float) -> float:
    return P / BW


def ideal_time(fl: float, nbytes: float, P: float, BW: float) -> float:
    return max(fl / P, nbytes / BW)


def onchip_bytes(BM: int, BN: int, BK: int, elem: int, acc_elem: int = 4, stages: int = 1,
                 with_acc: bool = True) -> int:
    inputs = stages * (BM * BK + BK * BN) * elem
    return inputs + (BM * BN * acc_elem if with_acc else 0)


def panel_a(BM: int, K: int, elem: int) -> int:
    return BM * K * elem


def panel_b(K: int, BN: int, elem: int) -> int:
    return K * BN * elem


def working_set_row_major(nn: int, pa: int, pb: int) -> int:
    return nn * pb + pa


def working_set_grouped(G: int, pa: int, pb: int) -> int:
    return G * pa + pb


def block_limit(available: float, per_block: float) -> int:
    return math.floor(available / per_block)


def waves_per_sm(grid: int, sms: int, blocks_per_sm: int) -> float:
    return grid / (sms * blocks_per_sm)


def tiles_per_program(num_tiles: int, P: int):
    """(min, max, number of programs that do max) for a persistent grid of P."""
    lo = num_tiles // P
    extra = num_tiles % P
    return lo, lo + (1 if extra else 0), (extra if extra else P)


# ---- per-XCD L2 locality model (this library's own) ------------------------------------

def l2_locality(nm: int, nn: int, grid: int, concurrent: int, xcds: int, order: str, G: int, remap: bool):
    """(cost, tiles): the first min(concurrent, grid) workgroups of a launch, workgroup
    w on XCD w mod xcds, each on the first tile of its schedule; cost = distinct
    (XCD, tile row) pairs + distinct (XCD, tile column) pairs.  Reuse = 1 - cost /
    (2 * tiles): the share of panel requests an XCD's L2 could serve from another
    tile in the same round."""
    from oracle import schedule as sch

    T = nm * nn
    rows, cols = set(), set()
    tiles = 0
    for w in range(min(concurrent, grid)):
        start = sch.xcd_remap(w, grid, xcds) if remap else w
        if start >= T:
            continue
        tm, tn = sch.grouped(start, nm, nn, G) if order == "grouped" else sch.row_major(start, nm, nn)
        rows.add((w % xcds, tm))
        cols.add((w % xcds, tn))
        tiles += 1
    return len(rows) + len(cols), tiles


AUTO_ORDER_CANDIDATES = (("grouped", 8, True), ("grouped", 4, True), ("grouped", 16, True),
                         ("row_major", 1, False), ("row_major", 1, True), ("grouped", 8, False),
                         ("grouped", 4, False), ("grouped", 16, False), ("grouped", 2, True),
                         ("grouped", 32, True), ("grouped", 2, False), ("grouped", 32, False))


def choose_order(nm: int, nn: int, grid: int, concurrent: int, xcds: int = 8):
    """The candidate (order, G, remap) of least locality cost, ties to the earlier
    candidate; grouped candidates with G > nm are skipped (same map as G = nm).
    Returns (order, G, remap, reuse in 1/1000, integer part)."""
    best = None
    for order, G, remap in AUTO_ORDER_CANDIDATES:
        if order == "grouped" and G > nm:
            continue
        cost, tiles = l2_locality(nm, nn, grid, concurrent, xcds, order, G, remap)
        if best is None or cost < best[0]:
            best = (cost, tiles, order, G, remap)
    cost, tiles, order, G, remap = best
    reuse_pm = (1000 - (1000 * cost) // (2 * tiles)) if tiles else 0
    return order, G, remap, reuse_pm
