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
