"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (from the acceptance bound of oracle.gemm): |C_gpu - C*| <= 2.5e-4 * S + 1e-6,
plus one unit in the last place of |C*| for 16-bit outputs.  Integer-valued
inputs make every fp32 accumulation exact, so there the GPU result must equal
the oracle's exact value rounded to the output type, bit for bit.
"""
import ctypes
import itertools
import re

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from tests.gpu_helpers import TORCH_OUT, round_to, sample_rows_cols, say, tile_sample, to_device, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_scheduling_amd as ts
else:  # collected on CPU-only hosts, never run there
    ts = None

TILES = ["64x64x32", "128x128x64", "256x256x64", "256x256x64w8", "256x256x64pp"]
IO = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]


def tile_dims(tile):
    """(BM, BN, BK) of a tile name such as "256x256x64w8"."""
    return tuple(int(v) for v in re.match(r"(\d+)x(\d+)x(\d+)", tile).groups())


def schedules(tile, P=256):
    out = []
    for (order, G), mode, remap in itertools.product([("row_major", 8), ("grouped", 8), ("grouped", 3)],
                                                      ["tiled", "persistent", "crosstile"], [False, True]):
        if tile == "256x256x64" and mode == "crosstile":
            continue   # no cross-tile kernel for that tile
        out.append(ts.Schedule(order=order, group_m=G, mode=mode, num_programs=0 if mode == "tiled" else P,
                               xcd_remap=remap, tile=tile))
    return out


def run(A, B, ab, c_dtype, sched, M, N, K):
    a, b = to_device(A, ab), to_device(B, ab)
    say(f"gemm {M}x{N}x{K} {ab}->{c_dtype} {sched.label()}")
    c = torch.full((M, N), float("nan"), dtype=TORCH_OUT[c_dtype], device="cuda")
    ts.gemm(a, b, out=c, schedule=sched)
    torch.cuda.synchronize()
    return c


def assert_accept(c_gpu, C, S, c_dtype, what=""):
    ok, worst, bad = og.accept(c_gpu, C, S, c_dtype)
    assert ok, f"{what}: {bad} outputs outside the bound (worst ratio {worst:.3g})"
    return worst


# ---- the ping-pong kernel against the 8-wave kernel ------------------------------------

@pytest.mark.parametrize("M,N,K", [(1024, 1536, 640), (1000, 1300, 448), (768, 512, 64)])
@pytest.mark.parametrize("ab,c_dtype", [("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("mode,P", [("tiled", 0), ("persistent", 5), ("persistent", 256), ("crosstile", 3)])
def test_pingpong_bit_identical_to_8_wave(M, N, K, ab, c_dtype, mode, P):
    # both kernels give every accumulator its K sub-steps in the same order, so
    # their outputs agree bit for bit, ragged tiles (edge path) included; and both
    # are checked against the oracle's bound
    A, B = workloads.pair(M, N, K, ab, "uniform", 520)
    outs = []
    for tile in ("256x256x64w8", "256x256x64pp"):
        s = ts.Schedule(order="grouped", group_m=3, mode=mode, num_programs=P, xcd_remap=True, tile=tile)
        outs.append(run(A, B, ab, c_dtype, s, M, N, K))
    assert torch.equal(outs[0], outs[1])
    C, S = og.gemm(A, B, ab, threads=4)
    assert_accept(to_f64(outs[1]), C, S, c_dtype, "ping-pong")


# ---- exactness with integer inputs ---------------------------------------------------

SHAPES = {"64x64x32": (200, 300, 130), "128x128x64": (300, 390, 200), "256x256x64": (600, 700, 260),
          "256x256x64w8": (600, 700, 260), "256x256x64pp": (600, 700, 260)}


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("ab,c_dtype", IO)
def test_integer_inputs_bit_exact(tile, ab, c_dtype):
    M, N, K = SHAPES[tile]
    A, B = workloads.pair(M, N, K, ab, "int", 500)
    C, _ = og.gemm(A, B, ab, threads=4)
    expect = round_to(C, c_dtype)
    second = "persistent" if tile == "256x256x64" else "crosstile"   # no cross-tile kernel for that tile
    for sched in (ts.Schedule(tile=tile), ts.Schedule(order="grouped", group_m=3, mode=second,
                                                      num_programs=5, tile=tile)):
        got = to_f64(run(A, B, ab, c_dtype, sched, M, N, K))
        bad = np.argwhere(got != expect)
        assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("tile", TILES)
def test_aligned_integer_inputs_bit_exact(tile):
    # whole tiles: the unmasked kernels
    bm, bn, bk = tile_dims(tile)
    M, N, K = 2 * bm, 3 * bn, 4 * bk
    A, B = workloads.pair(M, N, K, "f16", "int", 501)
    C, _ = og.gemm(A, B, "f16")
    assert ts.query(M, N, K, ts.Schedule(tile=tile))["masked"] == 0
    for mode in ("tiled", "persistent", "crosstile"):
        if tile == "256x256x64" and mode == "crosstile":
            continue   # no cross-tile kernel for that tile
        got = to_f64(run(A, B, "f16", "f32", ts.Schedule(mode=mode, num_programs=4, tile=tile), M, N, K))
        assert np.array_equal(got, C), mode


# ---- the 256^3 workload: 64x64x32 tiles, row-major, fp16 in, fp32 out ----------------

def test_square_256_f16_f32_full_oracle():
    w = workloads.SQUARE_256
    A, B = workloads.inputs(w)
    C, S = og.gemm(A, B, w.ab_dtype)
    sched = ts.Schedule(order="row_major", mode="tiled", tile="64x64x32")
    assert ts.query(w.M, w.N, w.K, sched, ts.TS_F16, ts.TS_F32)["grid"] == 16
    got = to_f64(run(A, B, w.ab_dtype, w.c_dtype, sched, w.M, w.N, w.K))
    worst = assert_accept(got, C, S, "f32", "256^3")
    say(f"256^3 worst |err|/bound = {worst:.3g}")


# ---- ragged shapes, every schedule, bit-identical across schedules -----------------

@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("ab,c_dtype", IO)
def test_ragged_every_schedule(tile, ab, c_dtype):
    bm, bn, bk = tile_dims(tile)
    M, N, K = 3 * bm + 17, 4 * bn + 9, 5 * bk + 11   # several tiles and a ragged tail in M, N, K
    A, B = workloads.pair(M, N, K, ab, "uniform" if ab == "f16" else "normal", 600)
    C, S = og.gemm(A, B, ab, threads=4)
    first = None
    for sched in schedules(tile, P=5):
        c = run(A, B, ab, c_dtype, sched, M, N, K)
        if first is None:
            first = c
            assert_accept(to_f64(c), C, S, c_dtype, sched.label())
        else:
            assert torch.equal(c, first), f"{sched.label()} differs from {schedules(tile)[0].label()}"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("ab,c_dtype", IO)
def test_ragged_word_aligned_rows(tile, ab, c_dtype):
    # K = 6 and N = 2 (mod 8): A and B rows are 4-byte but not 16-byte aligned, and
    # so are C rows of 16-bit outputs (fp32 rows are 8-byte aligned); the masked
    # loads and stores then move 4-byte pieces
    bm, bn, bk = tile_dims(tile)
    M, N, K = 2 * bm + 5, 3 * bn + 2, 4 * bk + 6
    A, B = workloads.pair(M, N, K, ab, "uniform" if ab == "f16" else "normal", 610)
    C, S = og.gemm(A, B, ab, threads=4)
    first = None
    for sched in schedules(tile, P=5):
        c = run(A, B, ab, c_dtype, sched, M, N, K)
        if first is None:
            first = c
            assert_accept(to_f64(c), C, S, c_dtype, sched.label())
        else:
            assert torch.equal(c, first), f"{sched.label()} differs from {schedules(tile)[0].label()}"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("ab,c_dtype", IO)
@pytest.mark.parametrize("n_tail", [8, 2], ids=["b16aligned", "b4aligned"])
def test_ragged_edge_paths(tile, ab, c_dtype, n_tail):
    # K a multiple of 8 with a partial last slice, M and N ragged: the direct-to-LDS
    # tiles zero-fill the edges (B rows 16-byte aligned when N = 0 mod 8, else only
    # 4-byte aligned); the 64-wide tile has no such pipeline and runs masked
    bm, bn, bk = tile_dims(tile)
    M, N, K = 2 * bm + 5, 3 * bn + n_tail, 4 * bk + 8
    expect_path = 1 if tile == "64x64x32" else 2
    assert ts.query(M, N, K, ts.Schedule(tile=tile))["masked"] == expect_path
    A, B = workloads.pair(M, N, K, ab, "uniform" if ab == "f16" else "normal", 620)
    C, S = og.gemm(A, B, ab, threads=4)
    first = None
    for sched in schedules(tile, P=5):
        c = run(A, B, ab, c_dtype, sched, M, N, K)
        if first is None:
            first = c
            assert_accept(to_f64(c), C, S, c_dtype, sched.label())
        else:
            assert torch.equal(c, first), f"{sched.label()} differs from {schedules(tile)[0].label()}"


@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64w8", "256x256x64pp"])
def test_edge_path_integer_inputs_bit_exact(tile):
    # exact integer products: any wrong or missing element (a tail chunk not zeroed,
    # a row past M read, a column past N stored) shows as a mismatch
    bm, bn, bk = tile_dims(tile)
    for (M, N, K) in ((bm + 1, bn + 2, bk + 8), (3 * bm - 7, 2 * bn + 8, 2 * bk + 56), (17, 30, 8)):
        A, B = workloads.pair(M, N, K, "f16", "int", 630)
        C, _ = og.gemm(A, B, "f16")
        for mode in ("tiled", "persistent", "crosstile"):
            got = to_f64(run(A, B, "f16", "f32", ts.Schedule(mode=mode, num_programs=3, tile=tile), M, N, K))
            assert np.array_equal(got, C), (M, N, K, mode)


# ---- the nested cross-tile kernels (at least 8 K steps) ------------------------------

@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64w8"])
@pytest.mark.parametrize("ab,c_dtype", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("shape,steps", [("whole", 8), ("edges", 10), ("whole", 9), ("edges", 11)])
def test_nested_crosstile_integer_inputs_bit_exact(tile, ab, c_dtype, shape, steps):
    # cross-tile mode with 8 to 11 K steps per tile runs a nested kernel: where a
    # program has more than one tile (P = 1 and 4; 15 on the 20 edge-shape tiles)
    # the one without the deferred wait, where each has one (P = 15 on the 15
    # whole-shape tiles, P = 32) the one whose last K step of a tile does not wait
    # for the next slice and whose post-epilogue wait counts the stores of the tile
    # just stored (edge tiles: none counted); with an odd count consecutive tiles
    # start on alternate slots; exact integer products, and bit-identical to the
    # persistent kernel
    bm, bn, bk = tile_dims(tile)
    if shape == "whole":
        M, N, K = 3 * bm, 5 * bn, steps * bk
    else:
        M, N, K = 3 * bm + 5, 4 * bn + 8, (steps - 1) * bk + 8
    A, B = workloads.pair(M, N, K, ab, "int", 640)
    C, _ = og.gemm(A, B, ab, threads=4)
    expect = round_to(C, c_dtype)
    assert ts.query(M, N, K, ts.Schedule(tile=tile))["masked"] == (0 if shape == "whole" else 2)
    for P in (1, 4, 15, 32):
        outs = []
        for mode in ("crosstile", "persistent"):
            s = ts.Schedule(order="grouped", group_m=2, mode=mode, num_programs=P, xcd_remap=True, tile=tile)
            got = run(A, B, ab, c_dtype, s, M, N, K)
            bad = np.argwhere(to_f64(got) != expect)
            assert bad.size == 0, f"{s.label()}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
            outs.append(got)
        assert torch.equal(outs[0], outs[1])


def test_nested_crosstile_random_inputs_back_to_back():
    # random fp16 inputs, ragged, 16 K steps per tile: two different products launched
    # back to back on one stream, each against the oracle's bound, and the auto
    # schedule (cross-tile) bit-identical to persistent
    outs = []
    for seed, (M, N, K) in ((650, (1300, 2048, 1024)), (651, (2000, 1100, 1000))):
        A, B = workloads.pair(M, N, K, "f16", "uniform", seed)
        C, S = og.gemm(A, B, "f16", threads=4)
        a, b = to_device(A, "f16"), to_device(B, "f16")
        q = ts.query(M, N, K, ts.Schedule(order="auto", mode="auto", tile="256x256x64w8"))
        assert q["mode"] == 2, q
        c = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ts.gemm(a, b, out=c, schedule=ts.Schedule(order="auto", mode="auto", tile="256x256x64w8"))
        outs.append((c, C, S, a, b, M, N))
    torch.cuda.synchronize()
    for c, C, S, a, b, M, N in outs:
        assert_accept(to_f64(c), C, S, "f16", f"{M}x{N}")
        p = torch.empty_like(c)
        ts.gemm(a, b, out=p, schedule=ts.Schedule(order="auto", mode="persistent", tile="256x256x64w8"))
        torch.cuda.synchronize()
        assert torch.equal(c, p)


# ---- the ragged bf16 workload at full size: all four schedules -----------------------

def test_ragged_bf16_5000x12290x1000_full_size():
    w = workloads.RAGGED_BF16
    A, B = workloads.inputs(w)
    rng = np.random.default_rng(7)
    base = None
    for sched in [ts.Schedule(tile="256x256x64"),
                  ts.Schedule(order="grouped", group_m=8, tile="256x256x64"),
                  ts.Schedule(order="grouped", group_m=8, mode="persistent", tile="256x256x64"),
                  ts.Schedule(order="grouped", group_m=8, mode="persistent", num_programs=3, xcd_remap=True,
                              tile="256x256x64"),
                  ts.Schedule(order="grouped", group_m=16, mode="persistent", xcd_remap=True, tile="256x256x64"),
                  # 8 waves: same per-element accumulation order, so bit-identical too
                  ts.Schedule(order="grouped", group_m=8, mode="tiled", xcd_remap=True, tile="256x256x64w8"),
                  ts.Schedule(order="grouped", group_m=8, mode="crosstile", tile="256x256x64w8")]:
        q = ts.query(w.M, w.N, w.K, sched, ts.TS_BF16, ts.TS_F32)
        # edges zero-filled by the direct-to-LDS loads, B's 4-byte aligned rows in 4-byte pieces
        assert q["masked"] == 2 and q["num_m_tiles"] == 20  # G = 8 leaves a short last group of 4 rows
        c = run(A, B, w.ab_dtype, w.c_dtype, sched, w.M, w.N, w.K)
        if base is None:
            base = c
        else:
            assert torch.equal(c, base), sched.label()
    rows, cols = sample_rows_cols(w.M, w.N, 256, 256, rng)
    for r in rows:
        C, S = og.gemm(A, B, w.ab_dtype, rows=(int(r), int(r) + 1))
        assert_accept(to_f64(base[r:r + 1]), C, S, w.c_dtype, f"row {r}")
    for cidx in cols:
        C, S = og.gemm(A, B, w.ab_dtype, cols=(int(cidx), int(cidx) + 1), threads=8)
        assert_accept(to_f64(base[:, cidx:cidx + 1]), C, S, w.c_dtype, f"col {cidx}")


# ---- the large square workloads, in the launch configurations the benchmark times ----

def _large(w, scheds, BM=256, BN=256):
    """Every schedule bit-identical to the first; then, on the first schedule's C,
    whole output tiles (every edge class, the first and last tile of each band of
    the grouped orders and of each XCD's run, 64 random tiles) and whole rows and
    columns (both edges of every tile-boundary class and random ones) against
    the oracle."""
    A, B = workloads.inputs(w)
    a, b = to_device(A, w.ab_dtype), to_device(B, w.ab_dtype)
    base = None
    for s in scheds:
        say(f"gemm {w.name} {s.label()}")
        c = torch.empty((w.M, w.N), dtype=TORCH_OUT[w.c_dtype], device="cuda")
        ts.gemm(a, b, out=c, schedule=s)
        torch.cuda.synchronize()
        if base is None:
            base = c
        else:
            assert torch.equal(c, base), s.label()
            del c
    rng = np.random.default_rng(11)
    tiles = tile_sample(w.M, w.N, BM, BN, rng)
    assert len(tiles) >= 64
    threads = max(1, min(16, og.max_threads()))
    worst = 0.0
    for tm, tn in tiles:
        r0, r1 = tm * BM, min(w.M, (tm + 1) * BM)
        c0, c1 = tn * BN, min(w.N, (tn + 1) * BN)
        C, S = og.gemm(A, B, w.ab_dtype, rows=(r0, r1), cols=(c0, c1), threads=threads)
        worst = max(worst, assert_accept(to_f64(base[r0:r1, c0:c1]), C, S, w.c_dtype, f"tile ({tm}, {tn})"))
    rows, cols = sample_rows_cols(w.M, w.N, BM, BN, rng, extra=3)
    for r in rows:
        C, S = og.gemm(A, B, w.ab_dtype, rows=(int(r), int(r) + 1), threads=threads)
        worst = max(worst, assert_accept(to_f64(base[r:r + 1]), C, S, w.c_dtype, f"row {r}"))
    for cidx in cols:
        C, S = og.gemm(A, B, w.ab_dtype, cols=(int(cidx), int(cidx) + 1), threads=threads)
        worst = max(worst, assert_accept(to_f64(base[:, cidx:cidx + 1]), C, S, w.c_dtype, f"col {cidx}"))
    say(f"{w.name}: {len(tiles)} tiles, {len(rows)} rows, {len(cols)} columns checked; "
        f"worst |err|/bound {worst:.3g}")


def test_8192x8192x4096_sampled():
    _large(workloads.SQ_8192, [ts.Schedule(order=o, group_m=8, mode=m, xcd_remap=r)
                               for o in ("row_major", "grouped") for m in ("tiled", "persistent")
                               for r in (False, True)])


def test_16384x16384x4096_sampled():
    _large(workloads.SQ_16384, [ts.Schedule(order=o, group_m=g, mode=m, xcd_remap=r)
                                for (o, g) in (("row_major", 8), ("grouped", 4), ("grouped", 8), ("grouped", 16))
                                for m in ("tiled", "persistent", "crosstile") for r in (False, True)])


def test_m_share_2048x16384x4096_sampled():
    # one GPU's share of an eight-way row split of the 16384 x 16384 x 4096 product
    _large(workloads.SHARE_M8, [ts.Schedule(order=o, group_m=8, mode=m, xcd_remap=r)
                                for (o, r) in (("row_major", False), ("grouped", True))
                                for m in ("tiled", "persistent", "crosstile")])


@pytest.mark.parametrize("w", [workloads.SQ_16384_BF16, workloads.SQ_16384_F32OUT], ids=lambda w: w.name)
def test_headline_shape_other_types_sampled(w):
    _large(w, [ts.Schedule(order="grouped", group_m=8, mode=m, xcd_remap=True) for m in ("persistent", "crosstile")])


def test_4096_cubed_sampled():
    _large(workloads.SQ_4096, [ts.Schedule(order=o, group_m=8, mode=m, xcd_remap=r, tile=t)
                               for (o, r) in (("row_major", False), ("grouped", True))
                               for m in ("tiled", "persistent", "crosstile") for t in ("auto",)])


@pytest.mark.parametrize("w", workloads.K_SWEEP, ids=lambda w: w.name)
def test_k_sweep_sampled(w):
    _large(w, [ts.Schedule(order="grouped", group_m=8, mode="persistent", xcd_remap=True),
               ts.Schedule(order="grouped", group_m=8, mode="crosstile", xcd_remap=True)])


# ---- edge cases ---------------------------------------------------------------------------

def test_empty_outputs_are_untouched():
    c = torch.full((4, 4), 7.0, device="cuda")
    a = torch.zeros((4, 8), dtype=torch.float16, device="cuda")
    b = torch.zeros((8, 4), dtype=torch.float16, device="cuda")
    assert ts.gemm_raw(a.data_ptr(), b.data_ptr(), c.data_ptr(), 0, 4, 8, c_dtype=ts.TS_F32) == ts.TS_OK
    assert ts.gemm_raw(a.data_ptr(), b.data_ptr(), c.data_ptr(), 4, 0, 8, c_dtype=ts.TS_F32) == ts.TS_OK
    torch.cuda.synchronize()
    assert (c == 7.0).all()


@pytest.mark.parametrize("mode", ["tiled", "persistent", "crosstile"])
@pytest.mark.parametrize("tile", TILES)
def test_k_zero_writes_zeros(mode, tile):
    if tile == "256x256x64" and mode == "crosstile":
        pytest.skip("no cross-tile kernel for the 4-wave 256 x 256 x 64 tile (rejected on the host)")
    a = torch.zeros((300, 0), dtype=torch.float16, device="cuda")
    b = torch.zeros((0, 270), dtype=torch.float16, device="cuda")
    c = torch.full((300, 270), float("nan"), dtype=torch.float16, device="cuda")
    say(f"K=0 {mode} {tile}")
    ts.gemm(a, b, out=c, schedule=ts.Schedule(mode=mode, num_programs=3, tile=tile))
    torch.cuda.synchronize()
    assert (c == 0).all()


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 777, 65), (513, 1, 33), (7, 9, 1), (65, 63, 8)])
def test_tiny_shapes(M, N, K):
    A, B = workloads.pair(M, N, K, "f16", "int", 70)
    C, _ = og.gemm(A, B, "f16")
    for tile in TILES:
        mode = "persistent" if tile == "256x256x64" else "crosstile"
        got = to_f64(run(A, B, "f16", "f32", ts.Schedule(mode=mode, num_programs=2, tile=tile), M, N, K))
        assert np.array_equal(got, C), tile


@pytest.mark.parametrize("tile", TILES)
def test_padded_and_unaligned_operands_with_canaries(tile):
    M, N, K = 333, 290, 150
    A, B = workloads.pair(M, N, K, "bf16", "int", 71)
    C, _ = og.gemm(A, B, "bf16")
    for pad, off in ((8, 0), (3, 1)):   # padded rows (aligned), then odd strides and odd offsets
        abuf = torch.zeros((M, K + pad + off), dtype=torch.bfloat16, device="cuda")
        bbuf = torch.zeros((K, N + pad + off), dtype=torch.bfloat16, device="cuda")
        a = abuf[:, off:off + K]
        b = bbuf[:, off:off + N]
        a.copy_(to_device(A, "bf16"))
        b.copy_(to_device(B, "bf16"))
        cbuf = torch.full((M + 4, N + 2 * pad + 2 * off + 2), -12345.0, device="cuda")
        c = cbuf[2:2 + M, pad + off:pad + off + N]
        say(f"strided {tile} pad={pad} off={off}")
        ts.gemm(a, b, out=c, schedule=ts.Schedule(order="grouped", group_m=2, mode="persistent",
                                                  num_programs=3, tile=tile))
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(c), C)
        guard = cbuf.clone()
        guard[2:2 + M, pad + off:pad + off + N] = -12345.0
        assert (guard == -12345.0).all(), "write outside C"


@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64", "256x256x64w8", "256x256x64pp"])
@pytest.mark.parametrize("N", [296, 290], ids=["b16aligned", "b4aligned"])
def test_edge_paths_padded_operands_with_canaries(tile, N):
    # padded row strides (8 elements) on the zero-filled-edge paths: the loads stop at
    # each matrix's last element, the stores stay inside C
    M, K, pad = 333, 152, 8
    A, B = workloads.pair(M, N, K, "bf16", "int", 73)
    C, _ = og.gemm(A, B, "bf16")
    abuf = torch.full((M, K + pad), 7.0, dtype=torch.bfloat16, device="cuda")
    bbuf = torch.full((K, N + pad), 7.0, dtype=torch.bfloat16, device="cuda")
    a, b = abuf[:, :K], bbuf[:, :N]
    a.copy_(to_device(A, "bf16"))
    b.copy_(to_device(B, "bf16"))
    cbuf = torch.full((M + 4, N + 2 * pad + 2), -12345.0, device="cuda")
    c = cbuf[2:2 + M, pad:pad + N]
    for mode in ("tiled", "persistent", "crosstile"):
        if tile == "256x256x64" and mode == "crosstile":
            continue   # no cross-tile kernel for that tile
        say(f"edge canaries {tile} N={N} {mode}")
        ts.gemm(a, b, out=c, schedule=ts.Schedule(order="grouped", group_m=2, mode=mode, num_programs=3,
                                                  tile=tile))
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(c), C), mode
        guard = cbuf.clone()
        guard[2:2 + M, pad:pad + N] = -12345.0
        assert (guard == -12345.0).all(), "write outside C"


def test_deterministic():
    A, B = workloads.pair(1000, 1100, 700, "f16", "uniform", 72)
    s = ts.Schedule(order="grouped", group_m=4, mode="crosstile", xcd_remap=True)
    c1 = run(A, B, "f16", "f16", s, 1000, 1100, 700)
    c2 = run(A, B, "f16", "f16", s, 1000, 1100, 700)
    assert torch.equal(c1, c2)


# ---- the clocked entry point: same product, plausible clock record -------------------

@pytest.mark.parametrize("mode", ["tiled", "persistent", "crosstile", "streamk"])
def test_gemm_clocked_matches_gemm(mode):
    M, N, K = 1024, 768, 512
    A, B = workloads.pair(M, N, K, "f16", "uniform", 777)
    a, b = to_device(A, "f16"), to_device(B, "f16")
    s = ts.Schedule(order="grouped", group_m=8, mode=mode, xcd_remap=True)
    say(f"gemm_clocked {M}x{N}x{K} {s.label()}")
    c0 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c1 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    ts.gemm(a, b, out=c0, schedule=s)
    rec = ts.gemm_clocked(a, b, c1, schedule=s)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    grid = ts.query(M, N, K, s)["grid"]
    assert rec.shape[0] == grid
    r = rec.cpu()
    assert bool((r[:, 1] > r[:, 0]).all()) and bool((r[:, 3] > r[:, 2]).all())
    clk = ts.clock_ghz(rec)
    say(f"clock {clk}")
    assert clk["programs"] == grid and 0.3 < clk["mean"] < 3.5


def test_gemm_clocked_rejects_short_record():
    M, N, K = 512, 512, 256
    a = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    b = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    c = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    rec = torch.zeros((1, 4), dtype=torch.int64, device="cuda")
    s = ts.Schedule(mode="tiled")
    assert ts.query(M, N, K, s)["grid"] > 1
    st = ts._lib.ts_gemm_clocked(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, K, 1, N, 1, N, 1,
                                 ts.TS_F16, ts.TS_F16, ctypes.byref(s._c()), 0, rec.data_ptr(), 1, None, 0)
    assert st == ts.TS_ERR_INVALID_ARG


def test_mfma_loop_probe_rate():
    tf = ts.mfma_loop_tflops(iters=4000, reps=2)
    say(f"mfma loop probe {tf:.1f} TFLOP/s")
    assert 200.0 < tf < 2600.0   # below the 2.4 GHz dense fp16 figure


@pytest.mark.parametrize("pattern", [0, 1, 2, 3])
def test_mfma_phase_probe_rate(pattern):
    tf = ts.mfma_phase_tflops(pattern, iters=2000, reps=2)
    say(f"mfma phase probe pattern {pattern}: {tf:.1f} TFLOP/s")
    assert 200.0 < tf < 2600.0


# ---- stream-K: split tiles, partial tiles added in a fixed order -----------------------

def _streamk_run(a, b, c, sched, ws):
    ts.gemm(a, b, out=c, schedule=sched, ws=ws)
    torch.cuda.synchronize()


def _streamk_ws(M, N, K, sched, ab, c_dtype):
    q = ts.query(M, N, K, sched, ts.TS_F16 if ab == "f16" else ts.TS_BF16,
                 {"f16": ts.TS_F16, "bf16": ts.TS_BF16, "f32": ts.TS_F32}[c_dtype])
    header = -(-(q["grid"] + 1) * 4 // 256) * 256
    ws = torch.zeros(max(q["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    return q, ws, header


def _streamk_header_clean(ws, q, header):
    h = ws[:header].view(torch.int32).cpu()
    assert int(h[:q["grid"]].abs().sum()) == 0, "flags not cleared"
    assert int(h[q["grid"]]) == 0, "a stream-K wait gave up"


@pytest.mark.parametrize("tile", ["64x64x32", "128x128x64", "256x256x64", "256x256x64w8"])
@pytest.mark.parametrize("ab,c_dtype", [("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("P", [5, 7, 64])
def test_streamk_ragged_against_oracle(tile, ab, c_dtype, P):
    bm, bn, bk = tile_dims(tile)
    M, N, K = 3 * bm + 17, 5 * bn + 9, 5 * bk + 11      # 4 x 6 = 24 tiles, ragged M, N, K
    A, B = workloads.pair(M, N, K, ab, "uniform" if ab == "f16" else "normal", 640)
    C, S = og.gemm(A, B, ab, threads=4)
    a, b = to_device(A, ab), to_device(B, ab)
    sched = ts.Schedule(order="grouped", group_m=3, mode="streamk", num_programs=P, xcd_remap=True, tile=tile)
    q, ws, header = _streamk_ws(M, N, K, sched, ab, c_dtype)
    assert q["workspace_bytes"] > 0    # 24 tiles on 5, 7 or 64 programs: 4, 3 or all 24 tiles split
    say(f"streamk {M}x{N}x{K} {ab}->{c_dtype} {sched.label()}")
    c1 = torch.full((M, N), float("nan"), dtype=TORCH_OUT[c_dtype], device="cuda")
    _streamk_run(a, b, c1, sched, ws)
    assert_accept(to_f64(c1), C, S, c_dtype, sched.label())
    _streamk_header_clean(ws, q, header)
    # the same again: bit-identical (partials are added in a fixed order)
    c2 = torch.full((M, N), float("nan"), dtype=TORCH_OUT[c_dtype], device="cuda")
    _streamk_run(a, b, c2, sched, ws)
    assert torch.equal(c1, c2)
    _streamk_header_clean(ws, q, header)


@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64w8"])
def test_streamk_integer_inputs_bit_exact(tile):
    # exact products and sums: any split of K gives the exact result
    bm, bn, bk = tile_dims(tile)
    for (M, N, K, P) in ((3 * bm + 5, 2 * bn + 8, 7 * bk + 8, 4), (2 * bm, 3 * bn, 6 * bk, 5), (17, 30, 8, 3)):
        A, B = workloads.pair(M, N, K, "f16", "int", 650)
        C, _ = og.gemm(A, B, "f16")
        sched = ts.Schedule(order="grouped", group_m=2, mode="streamk", num_programs=P, tile=tile)
        q, ws, header = _streamk_ws(M, N, K, sched, "f16", "f32")
        a, b = to_device(A, "f16"), to_device(B, "f16")
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        say(f"streamk int {M}x{N}x{K} P={P} {tile}")
        _streamk_run(a, b, c, sched, ws)
        assert np.array_equal(to_f64(c), C), (M, N, K, P)
        _streamk_header_clean(ws, q, header)


def test_streamk_without_split_equals_persistent():
    # whole rounds only: stream-K runs the persistent schedule, bit for bit
    M, N, K = 1024, 2048, 512            # 4 x 8 tiles of 256 x 256 on 8 programs
    A, B = workloads.pair(M, N, K, "f16", "uniform", 660)
    a, b = to_device(A, "f16"), to_device(B, "f16")
    s1 = ts.Schedule(order="grouped", group_m=8, mode="persistent", num_programs=8, xcd_remap=True)
    s2 = ts.Schedule(order="grouped", group_m=8, mode="streamk", num_programs=8, xcd_remap=True)
    assert ts.query(M, N, K, s2)["workspace_bytes"] == 0
    c1 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ts.gemm(a, b, out=c1, schedule=s1)
    ts.gemm(a, b, out=c2, schedule=s2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def test_streamk_ragged_bf16_full_size():
    # the 5000 x 12290 x 1000 bf16 workload: 980 tiles of 256 x 256 on 256 programs,
    # 212 of them split; every split tile and a sample of the others against the oracle
    w = workloads.RAGGED_BF16
    A, B = workloads.inputs(w)
    a, b = to_device(A, w.ab_dtype), to_device(B, w.ab_dtype)
    sched = ts.Schedule(order="grouped", group_m=8, mode="streamk", xcd_remap=True)
    q, ws, header = _streamk_ws(w.M, w.N, w.K, sched, w.ab_dtype, w.c_dtype)
    T, grid = q["num_tiles"], q["grid"]
    assert q["workspace_bytes"] > 0 and T % grid != 0
    say(f"streamk {w.name} {sched.label()} grid {grid}")
    c1 = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    _streamk_run(a, b, c1, sched, ws)
    _streamk_header_clean(ws, q, header)
    c2 = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    _streamk_run(a, b, c2, sched, ws)
    assert torch.equal(c1, c2)
    from oracle import schedule as osch
    nm, nn = q["num_m_tiles"], q["num_n_tiles"]
    split_ids = range(T - T % grid, T)
    tiles = {osch.grouped(t, nm, nn, 8) for t in split_ids}
    tiles |= set(tile_sample(w.M, w.N, 256, 256, np.random.default_rng(12), n_random=32))
    threads = max(1, min(16, og.max_threads()))
    worst = 0.0
    for tm, tn in sorted(tiles):
        r0, r1 = tm * 256, min(w.M, (tm + 1) * 256)
        c0, cc1 = tn * 256, min(w.N, (tn + 1) * 256)
        C, S = og.gemm(A, B, w.ab_dtype, rows=(r0, r1), cols=(c0, cc1), threads=threads)
        worst = max(worst, assert_accept(to_f64(c1[r0:r1, c0:cc1]), C, S, w.c_dtype, f"tile ({tm}, {tn})"))
    say(f"{w.name} stream-K: {len(tiles)} tiles checked, worst |err|/bound {worst:.3g}")
