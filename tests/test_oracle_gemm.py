"""Pins of the fp64 GEMM oracle against things other than itself.

Each test fixes the oracle to an independent fact: a library conversion or
product (numpy / torch), a closed form (identity, permutation, rank-1), a second
implementation (pure-Python loop), or an exact-arithmetic special case.
"""
import numpy as np
import pytest

import workloads
from oracle import gemm as og


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact small values -> 16-bit patterns through the library conversions."""
    x = np.asarray(x, dtype=np.float32)
    return workloads._round_to_bits(x, dtype).reshape(x.shape)


# ---- decoding: every bit pattern against the library conversions -----------------

def test_decode_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ours = og.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # subnormals and signed zero are part of the table above; spot-check a few
    assert og.decode(np.array([0x0001], np.uint16), "f16")[0] == 2.0 ** -24
    assert og.decode(np.array([0x3C00], np.uint16), "f16")[0] == 1.0
    assert og.decode(np.array([0xC000], np.uint16), "f16")[0] == -2.0


def test_decode_bf16_all_patterns():
    import torch

    bits = np.arange(65536, dtype=np.uint16)
    ours = og.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert og.decode(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert og.decode(np.array([0x0001], np.uint16), "bf16")[0] == 2.0 ** -133


# ---- the 4x4, 2x2-tile example against a hand expansion ------------------------------

def _golden_blocks(name):
    import os

    blocks, cur = {}, None
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line[0].isalpha():
                cur = blocks.setdefault(line, [])
            else:
                cur.append([float(v) for v in line.split()])
    return {k: np.array(v, dtype=np.float64) for k, v in blocks.items()}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_4x4_worked_shape_against_hand_expansion(dtype):
    # "Week-4 notes: Roofline and Tiling", section 5.1: 4x4 output, 2x2 tiles, K
    # slices of 2.  Values and expected sums are in tests/golden/gemm_4x4_int.txt.
    g = _golden_blocks("gemm_4x4_int.txt")
    C, S = og.gemm(_bits(g["A"], dtype), _bits(g["B"], dtype), dtype)
    assert np.array_equal(C, g["C"])
    assert np.array_equal(S, g["S"])
    # tile (0, 0) as the sum of its two K-slice products, each expanded by hand
    s0, s1 = og.gemm(_bits(g["A"][0:2, 0:2], dtype), _bits(g["B"][0:2, 0:2], dtype), dtype)[0], \
        og.gemm(_bits(g["A"][0:2, 2:4], dtype), _bits(g["B"][2:4, 0:2], dtype), dtype)[0]
    assert np.array_equal(s0, g["slice0"]) and np.array_equal(s1, g["slice1"])
    assert np.array_equal(s0 + s1, C[0:2, 0:2])
    # 2MNK = 128 floating point operations: 64 products, each followed by one add
    assert 2 * C.size * g["A"].shape[1] == 128


# ---- closed forms -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_identity_B_returns_A(dtype):
    A = workloads.matrix(37, 29, dtype, "uniform", 7)
    B = _bits(np.eye(29), dtype)
    C, S = og.gemm(A, B, dtype)
    a = og.decode(A, dtype)
    assert np.array_equal(C, a)
    assert np.array_equal(S, np.abs(a))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_permutation_B_permutes_columns(dtype):
    rng = np.random.default_rng(3)
    K = N = 41
    perm = rng.permutation(N)
    P = np.zeros((K, N))
    P[perm, np.arange(N)] = 1.0  # column j of C is column perm[j] of A
    A = workloads.matrix(23, K, dtype, "normal", 9)
    C, _ = og.gemm(A, _bits(P, dtype), dtype)
    assert np.array_equal(C, og.decode(A, dtype)[:, perm])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rank_one(dtype):
    # A = u s^T, B = t v^T  =>  C = (s . t) u v^T, exact with small integers
    rng = np.random.default_rng(11)
    M, N, K = 19, 23, 31
    u, s = rng.integers(-3, 4, M), rng.integers(-3, 4, K)
    t, v = rng.integers(-3, 4, K), rng.integers(-3, 4, N)
    A = _bits(np.outer(u, s), dtype)
    B = _bits(np.outer(t, v), dtype)
    C, S = og.gemm(A, B, dtype)
    assert np.array_equal(C, float(s @ t) * np.outer(u, v).astype(np.float64))
    assert np.array_equal(S, float(np.abs(s) @ np.abs(t)) * np.abs(np.outer(u, v)).astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_inputs_match_numpy_exactly(dtype):
    A = workloads.matrix(70, 130, dtype, "int", 21)
    B = workloads.matrix(130, 90, dtype, "int", 22)
    C, S = og.gemm(A, B, dtype)
    a, b = og.decode(A, dtype), og.decode(B, dtype)
    assert np.array_equal(C, a @ b)
    assert np.array_equal(S, np.abs(a) @ np.abs(b))


@pytest.mark.parametrize("dtype,dist", [("f16", "uniform"), ("bf16", "normal")])
def test_random_inputs_match_numpy_matmul(dtype, dist):
    M, N, K = 65, 47, 300
    A, B = workloads.pair(M, N, K, dtype, dist, 5)
    C, S = og.gemm(A, B, dtype, threads=4)
    a, b = og.decode(A, dtype), og.decode(B, dtype)
    ref = a @ b
    Sref = np.abs(a) @ np.abs(b)
    assert np.all(np.abs(C - ref) <= 1e-12 * Sref)
    assert np.allclose(S, Sref, rtol=1e-13, atol=0)
    assert np.all(S >= np.abs(C))


def test_zeros_and_empty_K():
    A = np.zeros((5, 7), np.uint16)
    B = np.zeros((7, 3), np.uint16)
    C, S = og.gemm(A, B, "f16")
    assert not C.any() and not S.any()
    C, S = og.gemm(np.zeros((4, 0), np.uint16), np.zeros((0, 6), np.uint16), "f16")
    assert C.shape == (4, 6) and not C.any() and not S.any()


def test_strided_views_follow_strides():
    # a transposed view of A (column-major storage) must give the same product
    dtype = "f16"
    A, B = workloads.pair(30, 20, 25, dtype, "uniform", 31)
    At = np.ascontiguousarray(A.T).T          # same values, strides (1, 30)
    Bt = np.ascontiguousarray(B.T).T
    C0, S0 = og.gemm(A, B, dtype)
    C1, S1 = og.gemm(At, Bt, dtype)
    assert np.array_equal(C0, C1) and np.array_equal(S0, S1)


def test_block_and_points_agree_with_full():
    dtype = "bf16"
    A, B = workloads.pair(40, 50, 60, dtype, "normal", 41)
    C, S = og.gemm(A, B, dtype)
    Cb, Sb = og.gemm(A, B, dtype, rows=(7, 33), cols=(11, 49))
    assert np.array_equal(Cb, C[7:33, 11:49]) and np.array_equal(Sb, S[7:33, 11:49])
    ii = np.array([0, 39, 5, 17])
    jj = np.array([49, 0, 5, 31])
    Cp, Sp = og.gemm_points(A, B, dtype, ii, jj)
    assert np.array_equal(Cp, C[ii, jj]) and np.array_equal(Sp, S[ii, jj])


# ---- brute force against a second implementation --------------------------------

def test_brute_force_tiny_shapes_against_python_loop():
    sizes = [1, 2, 3, 5, 8, 9, 15, 16, 17]
    rng = np.random.default_rng(77)
    for trial in range(60):
        M, N, K = (int(rng.choice(sizes)) for _ in range(3))
        dtype = "f16" if trial % 2 == 0 else "bf16"
        A, B = workloads.pair(M, N, K, dtype, "uniform", 1000 + trial)
        C, S = og.gemm(A, B, dtype)
        Cl, Sl = og.gemm_loop(og.decode(A, dtype).tolist(), og.decode(B, dtype).tolist())
        # same terms, same ascending order: identical bits
        assert np.array_equal(C, Cl), (M, N, K, dtype)
        assert np.array_equal(S, Sl), (M, N, K, dtype)


# ---- the acceptance bound -----------------------------------------------------------

def test_ulp_of_output_formats():
    assert og.ulp(np.array([1.0]), "f16")[0] == 2.0 ** -10
    assert og.ulp(np.array([1.5]), "f16")[0] == 2.0 ** -10
    assert og.ulp(np.array([2.0]), "f16")[0] == 2.0 ** -9
    assert og.ulp(np.array([0.0]), "f16")[0] == 2.0 ** -24
    assert og.ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert og.ulp(np.array([3.0]), "f32")[0] == 0.0
    # numpy's own spacing agrees for f16 normals
    x = np.array([0.7, 3.3, 100.0, 6e4], dtype=np.float16)
    assert np.array_equal(og.ulp(x.astype(np.float64), "f16"), np.spacing(x).astype(np.float64))


def test_accept_detects_planted_errors():
    dtype = "f16"
    A, B = workloads.pair(16, 16, 64, dtype, "uniform", 3)
    C, S = og.gemm(A, B, dtype)
    ok, worst, bad = og.accept(C.astype(np.float32), C, S, "f32")
    assert ok and bad == 0
    # rounding C to fp16 (RNE) stays inside the widened bound
    ok, _, _ = og.accept(C.astype(np.float16).astype(np.float64), C, S, "f16")
    assert ok
    # rounding the wrong way (one whole ulp off) is caught where S is small next to |C|
    ones = np.ones((4, 4))
    Sx = np.full((4, 4), 1.0)
    Cx = np.full((4, 4), 1.0 + 3 * 2.0 ** -11)      # halfway point between two fp16 values + 2^-11
    up = np.float64(np.float16(1.0 + 4 * 2.0 ** -11))
    down = np.float64(np.float16(1.0 + 2 * 2.0 ** -11))
    assert og.accept(np.full((4, 4), up), Cx, Sx * 0, "f16")[0]
    assert og.accept(np.full((4, 4), down), Cx, Sx * 0, "f16")[0]
    assert not og.accept(np.full((4, 4), up + 2.0 ** -10), Cx, Sx * 0, "f16")[0]
    assert not og.accept(ones * (down - 2.0 ** -10), Cx, Sx * 0, "f16")[0]
    # a dropped term is caught
    a, b = og.decode(A, dtype), og.decode(B, dtype)
    wrong = C - a[:, 5:6] * b[5:6, :]
    ok, _, bad = og.accept(wrong, C, S, "f32")
    assert not ok and bad > 0
    # NaN is caught
    Cn = C.copy()
    Cn[3, 4] = np.nan
    assert not og.accept(Cn, C, S, "f32")[0]
