"""Helpers for the GPU tests: move seeded bit arrays to the device, read results back."""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_IN = {"f16": torch.float16, "bf16": torch.bfloat16}
TORCH_OUT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(*args):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print("[case]", *args, file=sys.stderr, flush=True)


def to_device(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_IN[dtype])
    return t.to(device)


def to_f64(c: torch.Tensor) -> np.ndarray:
    return c.detach().float().cpu().numpy().astype(np.float64)


def round_to(c_exact: np.ndarray, c_dtype: str) -> np.ndarray:
    """Exact fp64 values rounded (RNE) to the output type, back in fp64."""
    t = torch.from_numpy(c_exact).to(TORCH_OUT[c_dtype])
    return t.to(torch.float64).numpy()


def sample_rows_cols(M: int, N: int, BM: int, BN: int, rng, extra: int = 6):
    """Rows and columns to check in full: both edges of every tile-boundary class
    (first, last, the last full tile and the ragged tail) plus random ones."""
    def pick(L, B):
        s = {0, 1, B - 1, B, L - 1, L - 2, (L // B) * B - 1, (L // B) * B}
        s |= {int(v) for v in rng.integers(0, L, extra)}
        return np.array(sorted(v for v in s if 0 <= v < L), dtype=np.int64)
    return pick(M, BM), pick(N, BN)


def tile_sample(M: int, N: int, BM: int, BN: int, rng, n_random: int = 64, groups=(4, 8, 16), P: int = 256,
                xcds: int = 8):
    """Output tiles to check element by element against the oracle:
    every corner and edge class of the tile grid (first / last tile row and
    column, the ragged tails), the first and last tile of every band of the
    grouped orders with G in ``groups``, the first and last tile that each XCD's
    workgroups compute in the persistent grouped + XCD-remap launch with P
    programs, and ``n_random`` seeded random tiles.  Returns sorted (tm, tn)."""
    from oracle import schedule as osch

    nm, nn = -(-M // BM), -(-N // BN)
    T = nm * nn
    tiles = {(0, 0), (0, nn - 1), (nm - 1, 0), (nm - 1, nn - 1), (nm // 2, nn // 2)}
    for G in groups:
        for first in range(0, T, min(G, nm) * nn):
            last = min(first + min(G, nm) * nn, T) - 1
            tiles.add(osch.grouped(first, nm, nn, min(G, nm)))
            tiles.add(osch.grouped(last, nm, nn, min(G, nm)))
    for G in groups:
        s = osch.Schedule(order=osch.GROUPED, group_m=min(G, nm), mode=osch.PERSISTENT,
                          num_programs=P, xcd_remap=True, xcds=xcds)
        Pe = osch.grid_size(T, s)
        for x in range(xcds):
            ids = [t for w in range(x, Pe, xcds) for t in osch.program_tiles(w, T, s)]
            if ids:
                tiles.add(osch.grouped(min(ids), nm, nn, min(G, nm)))
                tiles.add(osch.grouped(max(ids), nm, nn, min(G, nm)))
    for t in rng.choice(T, size=min(n_random, T), replace=False):
        tiles.add(osch.row_major(int(t), nm, nn))
    return sorted(tiles)
