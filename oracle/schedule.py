"""Tile-order schedules as plain enumerations -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  The GPU library computes every map below in closed form, with integer
division; this module builds each one instead by walking the tile grid in the
order the pages describe in words, and looks the answer up in the resulting
table.  The two forms share nothing, so a slip in either shows up as a
mismatch between the GPU trace and these tables.

Sources (cited by page title and section):
  * row-major order -- "(1/n) Triton matmul ... persistent kernel", naive tiled
    matmul listing: tile ids run along a row of output tiles, then move to the
    next row.
  * grouped order ("CTA swizzle") -- "(2/n) Triton matmul ... grouped ordering
    (CTA swizzle)", section "Implementation" and the prose around it: the tile
    rows are cut into bands of GROUP_SIZE_M rows (the last band holds whatever
    rows remain); ids fill one band completely before the next band starts,
    and inside a band they run down a tile column (M first), then move one
    column to the right.
  * persistent grid -- "(1/n) ...", naive persistent listing and its grid code:
    num_programs = min(CUs * programs_per_cu, num_tiles); program p takes tile
    ids p, p + P, p + 2P, ... below num_tiles.
  * flattened cross-tile loop -- "(3/n) ... cross tile pipelining", the merged
    loop.  Merging the tile loop and the K loop into one loop changes the
    control structure, not the sequence of (tile, K step) items: the merged loop
    visits exactly the concatenation of each tile's K steps, in the program's
    tile order.  The page sizes that loop as total = cdiv(num_tiles - start, P)
    * max(K_steps, 1) iterations; ``program_items`` checks its list against
    that count.
  * stream-K -- the persistent page names it as the follow-on for the tail of
    the persistent grid; how the tail is split is this library's own design,
    restated here from its definition: the first num_tiles - (num_tiles mod P)
    tiles (whole rounds of P programs) run as in the persistent mode; the K steps
    of the remaining tiles, listed tile by tile in tile-id order and k ascending
    inside a tile, are cut into P consecutive pieces whose lengths differ by at
    most one, longer pieces first (numpy.array_split's rule); piece r goes to
    program P - 1 - r, which runs it before its whole tiles.
  * XCD remap -- not on the pages.  A GPU with X chiplets (XCDs) deals the
    workgroups of a launch round-robin: workgroup w runs on chiplet w mod X.  The
    remap gives chiplet 0's workgroups the first run of logical ids, chiplet 1's
    the next run, and so on, each run in increasing w.

Parity pins: tests/test_oracle_schedule.py (bijection onto the tile grid,
G = 1 equals row-major, G >= num_m_tiles equals column-major, hand-worked
tables under tests/golden/, the persistent and flattened coverage invariants,
the program/tile counts the persistent page prints).
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

ROW_MAJOR = "row_major"
GROUPED = "grouped"
TILED = "tiled"
PERSISTENT = "persistent"
CROSSTILE = "crosstile"
STREAMK = "streamk"


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


@functools.lru_cache(maxsize=64)
def row_major_table(nm: int, nn: int):
    """Tile id -> (tile_m, tile_n): walk each tile row left to right, rows top to bottom."""
    table = []
    for tm in range(nm):
        for tn in range(nn):
            table.append((tm, tn))
    return tuple(table)


@functools.lru_cache(maxsize=256)
def grouped_table(nm: int, nn: int, G: int):
    """Tile id -> (tile_m, tile_n) of the grouped order: bands of G tile rows
    (the last band shorter if G does not divide nm); a band is filled column by
    column, each column top to bottom, before the next band starts."""
    if G < 1:
        raise ValueError("GROUP_SIZE_M must be >= 1")
    table = []
    band_top = 0
    while band_top < nm:
        band_rows = range(band_top, min(band_top + G, nm))
        for tn in range(nn):
            for tm in band_rows:
                table.append((tm, tn))
        band_top += G
    return tuple(table)


def row_major(t: int, nm: int, nn: int):
    return row_major_table(nm, nn)[t]


def grouped(t: int, nm: int, nn: int, G: int):
    return grouped_table(nm, nn, G)[t]


@functools.lru_cache(maxsize=256)
def xcd_remap_table(n: int, X: int = 8):
    """Launched workgroup w -> logical id: chiplet x's workgroups x, x+X, ...
    take one contiguous run of ids, the runs in chiplet order."""
    table = [None] * n
    nxt = 0
    for x in range(X):
        for w in range(x, n, X):
            table[w] = nxt
            nxt += 1
    return tuple(table)


def xcd_remap(w: int, n: int, X: int = 8) -> int:
    return xcd_remap_table(n, X)[w]


@dataclasses.dataclass(frozen=True)
class Schedule:
    order: str = ROW_MAJOR
    group_m: int = 8
    mode: str = TILED
    num_programs: int = 0   # persistent modes: requested grid (resolved by the caller)
    xcd_remap: bool = False
    xcds: int = 8


def tile_coords(t: int, nm: int, nn: int, s: Schedule):
    if s.order == ROW_MAJOR:
        return row_major(t, nm, nn)
    if s.order == GROUPED:
        return grouped(t, nm, nn, s.group_m)
    raise ValueError(s.order)


def grid_size(num_tiles: int, s: Schedule, ks: int = 1) -> int:
    """Programs launched: one per tile when tiled, min(P, num_tiles) when
    persistent, and min(P, num_tiles * max(ks, 1)) for stream-K (no more programs
    than (tile, K step) items)."""
    if s.mode == TILED:
        return num_tiles
    if s.num_programs < 1:
        raise ValueError("persistent schedules need num_programs >= 1")
    if s.mode == STREAMK:
        return min(s.num_programs, num_tiles * max(ks, 1))
    return min(s.num_programs, num_tiles)


def streamk_split(num_tiles: int, ks: int, P: int):
    """(whole tiles, pieces): the tiles run whole, and piece r of the split (tile
    id, k) items for r = 0 .. P-1."""
    split_tiles = num_tiles % P if ks > 0 else 0
    whole = num_tiles - split_tiles
    items = [(t, k) for t in range(whole, num_tiles) for k in range(ks)]
    pieces = [[items[i] for i in idx] for idx in np.array_split(np.arange(len(items)), P)]
    return whole, pieces


def program_tiles(p: int, num_tiles: int, s: Schedule):
    """Logical tile ids program p computes, in order."""
    P = grid_size(num_tiles, s)
    start = xcd_remap(p, P, s.xcds) if s.xcd_remap else p
    if s.mode == TILED:
        return [start]
    return list(range(start, num_tiles, P))


def program_items(p: int, nm: int, nn: int, ks: int, s: Schedule):
    """The (tile_m, tile_n, k_step) items program p works through, in order.

    Every tile keeps at least one K step (K = 0 still writes its tile)."""
    num_tiles = nm * nn
    ksp = max(ks, 1)
    items = []
    if s.mode == STREAMK:
        P = grid_size(num_tiles, s, ks)
        whole, pieces = streamk_split(num_tiles, ks, P)
        for t, k in pieces[P - 1 - p]:
            items.append(tile_coords(t, nm, nn, s) + (k,))
        start = xcd_remap(p, P, s.xcds) if s.xcd_remap else p
        for t in range(start, whole, P):
            tm, tn = tile_coords(t, nm, nn, s)
            items.extend((tm, tn, k) for k in range(ksp))
        return items
    for t in program_tiles(p, num_tiles, s):
        tm, tn = tile_coords(t, nm, nn, s)
        items.extend((tm, tn, k) for k in range(ksp))
    if s.mode == CROSSTILE:
        # the merged loop's iteration count on the cross-tile page
        P = grid_size(num_tiles, s)
        start = xcd_remap(p, P, s.xcds) if s.xcd_remap else p
        assert len(items) == cdiv(num_tiles - start, P) * ksp
    return items


def trace(M: int, N: int, K: int, BM: int, BN: int, BK: int, s: Schedule):
    """Rows (program, it, tile_m, tile_n, k_step) in the padded layout of the GPU trace.

    Program p owns rows [p * max_items, (p + 1) * max_items); rows beyond its
    item count hold -1 in every field.  max_items = cdiv(num_tiles, P) * max(ks, 1).
    """
    nm, nn, ks = cdiv(M, BM), cdiv(N, BN), cdiv(K, BK)
    num_tiles = nm * nn
    P = grid_size(num_tiles, s, ks) if num_tiles else 0
    ksp = max(ks, 1)
    per_program = [program_items(p, nm, nn, ks, s) for p in range(P)]
    if s.mode == STREAMK:
        max_items = max((len(x) for x in per_program), default=0)
    else:
        max_items = (cdiv(num_tiles, P) if P else 0) * ksp
    out = np.full((P * max_items, 5), -1, dtype=np.int32)
    for p in range(P):
        for it, (tm, tn, k) in enumerate(per_program[p]):
            out[p * max_items + it] = (p, it, tm, tn, k)
    return out
