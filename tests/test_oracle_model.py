"""Pins of the counting model: every number the pages print for it."""
import math
import os

import pytest

from oracle import model as m

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


def test_worked_4x4_example():
    g = _kv("worked_4x4.txt")
    M, N, K, BM, BN, BK, e = (int(g[k]) for k in ("M", "N", "K", "BM", "BN", "BK", "elem_bytes"))
    assert m.flops(M, N, K) == g["flops"]
    assert m.reads_no_reuse(M, N, K) == g["reads_no_reuse"]
    assert m.reads_tiled(M, N, K, BM, BN) == g["reads_tiled"]
    assert m.reads_ideal(M, N, K) == g["reads_ideal"]
    assert m.writes(M, N) * e == g["c_write_bytes"]
    b0 = m.traffic_bytes(m.reads_no_reuse(M, N, K), m.writes(M, N), e)
    b1 = m.traffic_bytes(m.reads_tiled(M, N, K, BM, BN), m.writes(M, N), e)
    assert (b0, b1) == (g["bytes_no_reuse"], g["bytes_tiled"])
    assert m.intensity(m.flops(M, N, K), b0) == pytest.approx(g["intensity_no_reuse"], abs=1e-12)
    assert m.intensity(m.flops(M, N, K), b1) == pytest.approx(g["intensity_tiled"], abs=1e-12)
    assert m.flops_step(BM, BN, BK) == g["flops_step"]
    assert m.flops_step(BM, BN, BK) * (K // BK) == g["flops_tile"]
    assert m.reads_step(BM, BN, BK) == g["reads_step"]
    # reuse factors 1 / 2 / 4: each element read serves that many outputs
    assert m.reads_no_reuse(M, N, K) // m.reads_tiled(M, N, K, BM, BN) == 2
    assert m.reads_no_reuse(M, N, K) // m.reads_ideal(M, N, K) == 4


def test_general_formulas_reduce_as_printed():
    M, N, K, BM, BN = 512, 768, 256, 64, 128
    assert m.reads_tiled(M, N, K, BM, BN) == M * N * K * (1 / BM + 1 / BN)
    assert m.reads_tile(BM, BN, K) * (M // BM) * (N // BN) == m.reads_tiled(M, N, K, BM, BN)
    T = 64  # BM = BN = T: reads 8MNK/T bytes in fp32, I ~ T/4
    r = m.reads_tiled(M, N, K, T, T) * 4
    assert r == 8 * M * N * K / T
    assert m.flops(M, N, K) / r == T / 4
    # ragged: only in-bounds elements
    assert m.reads_tiled(5, 3, 2, 4, 2) == 2 * (2 * 5 + 2 * 3)


def test_4096_fp32_roofline_table():
    # P = 20 TFLOP/s, BW = 1 TB/s, A = B = C = 4096^2 fp32, BM = BN = BK = T
    P, BW, n, e = 20e12, 1e12, 4096, 4
    F = m.flops(n, n, n)
    assert F == pytest.approx(1.37e11, abs=0.005e11)  # printed to three figures
    assert F / P * 1e3 == pytest.approx(6.87, abs=0.005)
    assert m.writes(n, n) * e / 1e9 == pytest.approx(0.067, abs=0.0005)
    assert m.ridge(P, BW) == 20
    rows = {  # T: (GB, I, bound TFLOP/s, time ms)
        None: (550, 0.25, 0.25, 550),
        32: (17.2, 7.97, 7.97, 17.2),
        64: (8.66, 15.9, 15.9, 8.66),
        128: (4.36, 31.5, 20, 6.87),
        "ideal": (0.20, 683, 20, 6.87),
    }
    for T, (gb, I, bound, ms) in rows.items():
        if T is None:
            reads = m.reads_no_reuse(n, n, n)
        elif T == "ideal":
            reads = m.reads_ideal(n, n, n)
        else:
            reads = m.reads_tiled(n, n, n, T, T)
        B = m.traffic_bytes(reads, m.writes(n, n), e)
        Ii = m.intensity(F, B)
        assert B / 1e9 == pytest.approx(gb, rel=0.01)
        assert Ii == pytest.approx(I, rel=0.01)
        assert m.roofline(P, BW, Ii) / 1e12 == pytest.approx(bound, rel=0.01)
        assert m.ideal_time(F, B, P, BW) * 1e3 == pytest.approx(ms, rel=0.01)
    # intensity stays just below T/4 because of the fixed C write
    for T in (32, 64, 128):
        Ii = m.intensity(F, m.traffic_bytes(m.reads_tiled(n, n, n, T, T), m.writes(n, n), e))
        assert Ii < T / 4


def test_onchip_bytes_table():
    KB = 1024
    assert m.onchip_bytes(32, 32, 32, 4) == 12 * KB
    assert m.onchip_bytes(64, 64, 64, 4) == 48 * KB
    assert m.onchip_bytes(128, 128, 128, 4) == 192 * KB
    assert m.onchip_bytes(128, 128, 128, 4, with_acc=False) == 128 * KB
    assert m.onchip_bytes(128, 128, 128, 4, stages=2, with_acc=False) == 256 * KB
    assert m.onchip_bytes(128, 128, 32, 4, with_acc=False) == 32 * KB
    # accumulator of 128x128 fp32 = 16384 registers = 64 per thread over 256 threads
    assert 128 * 128 // 256 == 64
    # fp16 stage buffer of the Triton kernels (128x64x32): 12288 B, three stages 36864 B
    assert m.onchip_bytes(128, 64, 32, 2, with_acc=False) == 12288
    assert m.onchip_bytes(128, 64, 32, 2, stages=3, with_acc=False) == 36864


def test_panel_and_working_set_sizes():
    MiB = 1 << 20
    pa, pb = m.panel_a(128, 4096, 2), m.panel_b(4096, 64, 2)
    assert (pa, pb) == (1 * MiB, MiB // 2)
    assert m.working_set_row_major(8192 // 64, pa, pb) == 65 * MiB
    assert m.working_set_row_major(16384 // 64, pa, pb) == 129 * MiB
    assert m.working_set_grouped(8, pa, pb) == 8.5 * MiB


def test_block_limit_and_wave_arithmetic():
    assert 174 * 128 == 22272
    assert 65536 / 22272 == pytest.approx(2.94, abs=0.005)
    assert m.block_limit(65536, 174 * 128) == 2
    assert 102400 / (36864 + 1024) == pytest.approx(2.70, abs=0.005)
    assert m.block_limit(100 * 1024, 36864 + 1024) == 2
    assert m.block_limit(48, 4) == 12
    assert 8 / 48 == pytest.approx(0.1667, abs=1e-4)
    assert m.waves_per_sm(2048, 170, 2) == pytest.approx(6.02, abs=0.005)
    assert m.waves_per_sm(170, 170, 2) == 0.5
    assert m.waves_per_sm(340, 170, 2) == 1.0
    assert m.tiles_per_program(2048, 340) == (6, 7, 8)


def test_page_timings_are_2mnk_over_t():
    # every time / TFLOPS pair on the swizzle page satisfies TFLOPS = 2MNK / t
    for (M, N, K), ms, tf in [((8192, 8192, 4096), 2.4443, 224.91),
                              ((8192, 8192, 4096), 2.5502, 215.57),
                              ((16384, 16384, 4096), 11.6640, 188.53),
                              ((16384, 16384, 4096), 10.4398, 210.64),
                              ((4096, 4096, 4096), 0.6448, 213.16)]:
        assert m.flops(M, N, K) / (ms * 1e-3) / 1e12 == pytest.approx(tf, abs=0.02)
    assert math.isclose(1 - 10.4398 / 11.6640, 0.105, abs_tol=0.001)


# ---- per-XCD L2 locality model -------------------------------------------------------------

def test_l2_locality_hand_worked_4x4_grid_on_4_xcds():
    # 4 x 4 tiles, 16 workgroups on 4 XCDs (4 tiles each), worked by hand:
    # row-major: XCD x holds tile column x (4 rows + 1 column = 5 each, cost 20);
    # row-major + remap: tile row x (cost 20); grouped G = 2 (with or without the
    # remap): a 2 x 2 block per XCD (2 + 2 = 4 each, cost 16); G = 4 (column-major):
    # cost 20 either way
    L = m.l2_locality
    assert L(4, 4, 16, 16, 4, "row_major", 1, False) == (20, 16)
    assert L(4, 4, 16, 16, 4, "row_major", 1, True) == (20, 16)
    assert L(4, 4, 16, 16, 4, "grouped", 2, False) == (16, 16)
    assert L(4, 4, 16, 16, 4, "grouped", 2, True) == (16, 16)
    assert L(4, 4, 16, 16, 4, "grouped", 4, False) == (20, 16)
    assert L(4, 4, 16, 16, 4, "grouped", 4, True) == (20, 16)
    # the choice: G = 8 and 16 are skipped (G > nm), G = 4 + remap costs 20, the
    # first candidate of cost 16 is G = 2 + remap: reuse 1 - 16/32
    assert m.choose_order(4, 4, 16, 16, 4) == ("grouped", 2, True, 500)


@pytest.mark.parametrize("bm,concurrent,expect", [
    # reuse fractions computed for the 16384 x 16384 grid when the build was planned
    (256, 256, {("row_major", 1, False): 0.81, ("row_major", 1, True): 0.48, ("grouped", 4, False): 0.48,
                ("grouped", 4, True): 0.81, ("grouped", 8, False): 0.48, ("grouped", 8, True): 0.81,
                ("grouped", 16, False): 0.72, ("grouped", 16, True): 0.72}),
    (128, 512, {("row_major", 1, False): 0.84, ("row_major", 1, True): 0.49, ("grouped", 4, False): 0.49,
                ("grouped", 4, True): 0.84, ("grouped", 8, False): 0.49, ("grouped", 8, True): 0.88,
                ("grouped", 16, False): 0.73, ("grouped", 16, True): 0.84}),
])
def test_l2_locality_planned_fractions_for_16384(bm, concurrent, expect):
    nm = nn = 16384 // bm
    for (order, G, remap), frac in expect.items():
        cost, tiles = m.l2_locality(nm, nn, concurrent, concurrent, 8, order, G, remap)
        assert round(1 - cost / (2 * tiles), 2) == frac, (order, G, remap)
