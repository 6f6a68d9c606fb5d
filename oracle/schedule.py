"""Tile-order schedules as plain integer functions -- TEST INFRASTRUCTURE ONLY.

Sources (cited by page title and section):
  * row-major order -- "(1/n) Triton matmul ... persistent kernel", naive tiled
    matmul listing: tile_m = tile_id // num_n_tiles, tile_n = tile_id % num_n_tiles.
  * grouped order ("CTA swizzle") -- "(2/n) Triton matmul ... grouped ordering
    (CTA swizzle)", section "Implementation" (the three SWIZZLE steps): groups
    of GROUP_SIZE_M tile rows, the last group possibly shorter, and inside a
    group the M coordinate advances first.
  * persistent grid -- "(1/n) ...", naive persistent listing and its grid code:
    num_programs = min(CUs * programs_per_cu, num_tiles); program p takes tile
    ids p, p + P, p + 2P, ... below num_tiles.
  * flattened cross-tile loop -- "(3/n) ... cross tile pipelining", the merged
    loop: outer_iters = cdiv(num_tiles - start, P), total = outer_iters *
    max(K_steps, 1), tile set-up at k == 0, store at k == K_steps - 1, then k
    wraps to 0.
  * XCD remap -- not on the pages.  A bijection on [0, n) that sends the ids a
    GPU with X chiplets (XCDs) deals round-robin to chiplet x (w = x, x+X, ...)
    to one contiguous run of logical ids: w -> (w % X) * q + min(w % X, r) + w // X,
    q = n // X, r = n % X.

Parity pins: tests/test_oracle_schedule.py (bijection onto the tile grid,
G = 1 equals row-major, G >= num_m_tiles equals column-major, hand-worked
tables under tests/golden/, the persistent and flattened coverage invariants,
the program/tile counts the persistent page prints).
"""
from __future__ import annotations

import dataclasses

import numpy as np

ROW_MAJOR = "row_major"
GROUPED = "grouped"
TILED = "tiled"
PERSISTENT = "persistent"
CROSSTILE = "crosstile"


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def row_major(t: int, nm: int, nn: int):
    return t // nn, t % nn


def grouped(t: int, nm: int, nn: int, G: int):
    if G < 1:
        raise ValueError("GROUP_SIZE_M must be >= 1")
    num_tiles_in_group = G * nn
    group_id = t // num_tiles_in_group
    tile_id_in_group = t % num_tiles_in_group
    first_tile_m = group_id * G
    group_size_m = min(G, nm - first_tile_m)
    return first_tile_m + tile_id_in_group % group_size_m, tile_id_in_group // group_size_m


def xcd_remap(w: int, n: int, X: int = 8) -> int:
    q, r = n // X, n % X
    x = w % X
    return x * q + min(x, r) + w // X


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


def grid_size(num_tiles: int, s: Schedule) -> int:
    """Programs launched: one per tile when tiled, else min(P, num_tiles)."""
    if s.mode == TILED:
        return num_tiles
    if s.num_programs < 1:
        raise ValueError("persistent schedules need num_programs >= 1")
    return min(s.num_programs, num_tiles)


def program_items(p: int, nm: int, nn: int, ks: int, s: Schedule):
    """The (tile_m, tile_n, k_step) items program p works through, in order."""
    num_tiles = nm * nn
    P = grid_size(num_tiles, s)
    start = xcd_remap(p, P, s.xcds) if s.xcd_remap else p
    ksp = max(ks, 1)
    if s.mode == TILED:
        tiles = [start]
    else:
        tiles = list(range(start, num_tiles, P))
    items = []
    if s.mode == CROSSTILE:
        # one merged loop: iteration i -> tile (start + (i // ksp) * P), k = i % ksp
        total = cdiv(num_tiles - start, P) * ksp
        k = 0
        tile = start
        for _ in range(total):
            items.append(tile_coords(tile, nm, nn, s) + (k,))
            if k == ksp - 1:
                k = 0
                tile += P
            else:
                k += 1
    else:
        for t in tiles:
            tm, tn = tile_coords(t, nm, nn, s)
            for k in range(ksp):
                items.append((tm, tn, k))
    return items


def trace(M: int, N: int, K: int, BM: int, BN: int, BK: int, s: Schedule):
    """Rows (program, it, tile_m, tile_n, k_step) in the padded layout of the GPU trace.

    Program p owns rows [p * max_items, (p + 1) * max_items); rows beyond its
    item count hold -1 in every field.  max_items = cdiv(num_tiles, P) * max(ks, 1).
    """
    nm, nn, ks = cdiv(M, BM), cdiv(N, BN), cdiv(K, BK)
    num_tiles = nm * nn
    P = grid_size(num_tiles, s) if num_tiles else 0
    ksp = max(ks, 1)
    max_items = (cdiv(num_tiles, P) if P else 0) * ksp
    out = np.full((P * max_items, 5), -1, dtype=np.int32)
    for p in range(P):
        for it, (tm, tn, k) in enumerate(program_items(p, nm, nn, ks, s)):
            out[p * max_items + it] = (p, it, tm, tn, k)
    return out
