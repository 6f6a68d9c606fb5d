"""Seeded synthetic inputs for the tiled-GEMM workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds input generation only: no part of the matrix product, the
tile maps or any other arithmetic of the method lives here.

Every matrix is produced on the host as the raw 16-bit storage pattern of an
IEEE binary16 ("f16") or bfloat16 ("bf16") value, held in a numpy ``uint16``
array of shape (rows, cols), row-major. Both sides read exactly these bits: the
oracle decodes them itself, the GPU path copies them to device memory.

Recipes (seeded numpy PCG64 generator, float32 draw, then round to nearest even):
  * ``uniform``  : 2*U[0,1) - 1, i.e. values in [-1, 1)
  * ``normal``   : standard normal N(0, 1)
  * ``int``      : integers drawn uniformly from {-2, ..., 2} (exact in f16/bf16)
The A matrix of a workload uses ``seed`` and the B matrix ``seed + 1``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

DTYPES = ("f16", "bf16")


def _round_to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the 16-bit storage type (RNE) and return the bits."""
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch  # library rounding to bfloat16 (round to nearest even)

        t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def matrix(rows: int, cols: int, dtype: str, dist: str, seed: int) -> np.ndarray:
    """Return a (rows, cols) uint16 array holding seeded values of ``dtype``."""
    rng = np.random.default_rng(seed)
    shape = (rows, cols)
    if dist == "uniform":
        x = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    elif dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "int":
        x = rng.integers(-2, 3, size=shape).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(_round_to_bits(x, dtype))


def pair(M: int, N: int, K: int, dtype: str, dist: str, seed: int):
    """Return (A bits [M,K], B bits [K,N]) for one workload."""
    return matrix(M, K, dtype, dist, seed), matrix(K, N, dtype, dist, seed + 1)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM shape the pages measure, with its input recipe."""

    name: str
    M: int
    N: int
    K: int
    ab_dtype: str  # "f16" or "bf16"
    c_dtype: str   # "f16", "bf16" or "f32"
    dist: str
    seed: int


# The workloads (shapes, value distributions, output types); seeds are 1000 + index.
SQUARE_256 = Workload("gemm_256x256x256_f16_f32", 256, 256, 256, "f16", "f32", "uniform", 1000)
SQ_8192 = Workload("gemm_8192x8192x4096_f16", 8192, 8192, 4096, "f16", "f16", "uniform", 1001)
SQ_16384 = Workload("gemm_16384x16384x4096_f16", 16384, 16384, 4096, "f16", "f16", "uniform", 1002)
K_SWEEP = tuple(
    Workload(f"gemm_16384x16384x{k}_f16_ksweep", 16384, 16384, k, "f16", "f16", "uniform", 1003)
    for k in (128, 512, 1024, 2048, 4096)
)
RAGGED_BF16 = Workload("gemm_5000x12290x1000_bf16_f32", 5000, 12290, 1000, "bf16", "f32", "normal", 1004)
# One GPU's share of the 16384 x 16384 x 4096 product split eight ways by rows of A and C.
SHARE_M8 = Workload("gemm_2048x16384x4096_f16_mshare8", 2048, 16384, 4096, "f16", "f16", "uniform", 1005)

# The 4096-cubed product the grouped-ordering page also measures.
SQ_4096 = Workload("gemm_4096x4096x4096_f16", 4096, 4096, 4096, "f16", "f16", "uniform", 1006)

# The headline shape with bf16 inputs and output, and with fp16 inputs and fp32 output.
SQ_16384_BF16 = Workload("gemm_16384x16384x4096_bf16", 16384, 16384, 4096, "bf16", "bf16", "uniform", 1007)
SQ_16384_F32OUT = Workload("gemm_16384x16384x4096_f16_f32", 16384, 16384, 4096, "f16", "f32", "uniform", 1008)

ALL = (SQUARE_256, SQ_8192, SQ_16384) + K_SWEEP + (RAGGED_BF16, SHARE_M8, SQ_4096, SQ_16384_BF16, SQ_16384_F32OUT)


def inputs(w: Workload):
    """Seeded (A bits, B bits) for workload ``w``."""
    return pair(w.M, w.N, w.K, w.ab_dtype, w.dist, w.seed)
