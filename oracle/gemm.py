"""fp64 oracle for C = A @ B on fp16/bf16 inputs -- TEST INFRASTRUCTURE ONLY.

Follows the plain definition in "Week-4 notes: Roofline and Tiling" (section 1:
C[M,N] = A[M,K] @ B[K,N], every output a sum of K products, 2MNK FLOPs), with
the fp32 accumulator of the Triton matmul pages ("(1/n) ... persistent kernel",
naive tiled matmul listing) replaced by fp64 so that the oracle is exact up to
fp64 summation.  The heavy loops are in ``ref_gemm.c``; ``gemm_loop`` is a
second, pure-Python implementation for tiny shapes.

Parity pins (tests/test_oracle_gemm.py): a 4x4 product with 2x2 output tiles, the
shape of the worked example of section 5.1, against a hand expansion
(tests/golden/gemm_4x4_int.txt; the page's own matrix values did not survive),
identity and permutation B, rank-1 inputs, small-integer inputs against
numpy.matmul, zeros and K = 0, brute force against ``gemm_loop``, and the
decoders against numpy/torch conversions.

Acceptance (``accept``): |C_gpu - C*| <= 2.5e-4 * S + 1e-6 elementwise, where S
= sum_k |a_ik b_kj|; 2.5e-4 covers the worst-case fp32 summation error
K * 2^-24 for K <= 4096.  A 16-bit output adds the error of one round-to-
nearest-even conversion of the fp32 accumulator x to the output type: half a
unit in the last place at |x|.  |x| is at most |C*| + e with e = 2.5e-4 * S +
1e-6, so the added term is ulp_out(|C*| + e) / 2 (the ulp is taken at the larger
magnitude so that an accumulator just above a power of two is covered).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtsoracle.so")
_DTYPE_CODE = {"f16": 1, "bf16": 2}
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b

            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ts_oracle_decode.argtypes = [_p, _i64, ctypes.c_int, _p]
        lib.ts_oracle_gemm_block.argtypes = [_p, _p, ctypes.c_int] + [_i64] * 11 + [_p, _p, _i64, ctypes.c_int]
        lib.ts_oracle_gemm_points.argtypes = [_p, _p, ctypes.c_int] + [_i64] * 7 + [_p, _p, _i64, _p, _p, ctypes.c_int]
        lib.ts_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ts_oracle_max_threads())


def _u16(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("oracle inputs are 2-D uint16 bit arrays")
    return x


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of 16-bit patterns (any shape)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    rc = _load().ts_oracle_decode(b.ctypes.data, b.size, _DTYPE_CODE[dtype], out.ctypes.data)
    if rc != 0:
        raise ValueError("decode failed")
    return out


def _strides(x: np.ndarray):
    return x.strides[0] // 2, x.strides[1] // 2


def gemm(A: np.ndarray, B: np.ndarray, dtype: str, rows=None, cols=None, threads: int = 1):
    """(C, S) in fp64 for the block rows x cols of A @ B (default: all of it).

    A is (M, K), B is (K, N), both uint16 bit arrays of ``dtype``; any strides.
    """
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    i0, i1 = rows if rows is not None else (0, M)
    j0, j1 = cols if cols is not None else (0, N)
    C = np.zeros((max(i1 - i0, 0), max(j1 - j0, 0)), dtype=np.float64)
    S = np.zeros_like(C)
    s_am, s_ak = _strides(A)
    s_bk, s_bn = _strides(B)
    rc = _load().ts_oracle_gemm_block(A.ctypes.data, B.ctypes.data, _DTYPE_CODE[dtype],
                                      M, N, K, s_am, s_ak, s_bk, s_bn, i0, i1, j0, j1,
                                      C.ctypes.data, S.ctypes.data, C.shape[1], int(threads))
    if rc != 0:
        raise ValueError(f"oracle gemm failed ({rc})")
    return C, S


def gemm_points(A: np.ndarray, B: np.ndarray, dtype: str, ii, jj, threads: int = 1):
    """(C, S) in fp64 at the scattered outputs (ii[p], jj[p])."""
    A, B = _u16(A), _u16(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    C = np.zeros(ii.shape, dtype=np.float64)
    S = np.zeros_like(C)
    s_am, s_ak = _strides(A)
    s_bk, s_bn = _strides(B)
    rc = _load().ts_oracle_gemm_points(A.ctypes.data, B.ctypes.data, _DTYPE_CODE[dtype],
                                       M, N, K, s_am, s_ak, s_bk, s_bn,
                                       ii.ctypes.data, jj.ctypes.data, ii.size,
                                       C.ctypes.data, S.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle gemm_points failed ({rc})")
    return C, S


def gemm_loop(a: np.ndarray, b: np.ndarray):
    """Pure-Python triple loop on already-decoded fp64 matrices (tiny shapes only).

    C[i][j] = sum over k, ascending, of a[i][k] * b[k][j]; S likewise with |.|.
    """
    M, K = len(a), (len(a[0]) if len(a) else 0)
    N = len(b[0]) if len(b) else 0
    C = [[0.0] * N for _ in range(M)]
    S = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            c = 0.0
            s = 0.0
            for k in range(K):
                p = float(a[i][k]) * float(b[k][j])
                c += p
                s += abs(p)
            C[i][j] = c
            S[i][j] = s
    return np.array(C, dtype=np.float64).reshape(M, N), np.array(S, dtype=np.float64).reshape(M, N)


# ---- acceptance ---------------------------------------------------------------------

REL = 2.5e-4
ABS = 1e-6
# mantissa bits (without the implicit bit) and the smallest normal exponent of each output type
_FMT = {"f16": (10, -14), "bf16": (7, -126)}


def ulp(x: np.ndarray, c_dtype: str) -> np.ndarray:
    """Spacing of the output format at |x| (one unit in the last place)."""
    if c_dtype == "f32":
        return np.zeros_like(np.asarray(x, dtype=np.float64))
    mbits, emin = _FMT[c_dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(ax))          # -inf at zero
    e = np.maximum(e, emin)                # subnormal range keeps the spacing of 2^emin
    return np.ldexp(1.0, (e - mbits).astype(np.int64))


def bound(C_ref: np.ndarray, S: np.ndarray, c_dtype: str) -> np.ndarray:
    e = REL * S + ABS
    return e + 0.5 * ulp(np.abs(C_ref) + e, c_dtype)


def accept(C_gpu: np.ndarray, C_ref: np.ndarray, S: np.ndarray, c_dtype: str):
    """Return (ok, worst |err|/bound, number of violations)."""
    err = np.abs(np.asarray(C_gpu, dtype=np.float64) - C_ref)
    b = bound(C_ref, S, c_dtype)
    finite = np.isfinite(err)
    ratio = np.where(finite, err / b, np.inf)
    bad = int(np.count_nonzero(~(ratio <= 1.0)))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bad == 0, worst, bad
