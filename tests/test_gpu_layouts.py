"""Operand layouts through the element strides of the pages' kernel signature:
A stored [M][K] or [K][M], B stored [K][N] or [N][K] (NN, NT, TN, TT), against
the oracle, which follows any strides."""
import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from tests.gpu_helpers import TORCH_OUT, say, tile_sample, to_device, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_scheduling_amd as ts
else:
    ts = None

LAYOUTS = ["NN", "NT", "TN", "TT"]


def operands(A, B, ab, layout):
    """Device views with A's and B's logical values in the requested storage order."""
    a = to_device(A, ab) if layout[0] == "N" else to_device(np.ascontiguousarray(A.T), ab).t()
    b = to_device(B, ab) if layout[1] == "N" else to_device(np.ascontiguousarray(B.T), ab).t()
    assert (a.stride(1) == 1) == (layout[0] == "N") and (b.stride(1) == 1) == (layout[1] == "N")
    return a, b


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("tile", ["64x64x32", "128x128x64", "256x256x64", "256x256x64w8", "256x256x64pp"])
@pytest.mark.parametrize("whole", [True, False], ids=["whole", "ragged"])
def test_layouts_integer_inputs_bit_exact(layout, tile, whole):
    bm, bn, bk = (int(v) for v in tile[:-2 if tile[-2:] in ("w8", "pp") else None].split("x"))
    M, N, K = (2 * bm, 3 * bn, 4 * bk) if whole else (2 * bm + 5, 3 * bn + 3, 3 * bk + 7)
    A, B = workloads.pair(M, N, K, "f16", "int", 800)
    C, _ = og.gemm(A, B, "f16")
    a, b = operands(A, B, "f16", layout)
    for mode in ("tiled", "persistent", "crosstile", "streamk"):
        if tile == "256x256x64" and mode == "crosstile":
            continue
        s = ts.Schedule(order="grouped", group_m=2, mode=mode, num_programs=5, tile=tile)
        say(f"layout {layout} {M}x{N}x{K} {s.label()}")
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ts.gemm(a, b, out=c, schedule=s)
        torch.cuda.synchronize()
        got = to_f64(c)
        bad = np.argwhere(got != C)
        assert bad.size == 0, f"{layout} {mode}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64w8"])
@pytest.mark.parametrize("steps", [8, 9])
def test_layouts_nested_crosstile_bit_exact(layout, tile, steps):
    # 8 or 9 K steps per tile: the cross-tile mode runs the nested kernel on every layout
    bm, bn, bk = (int(v) for v in tile[:-2 if tile[-2:] in ("w8", "pp") else None].split("x"))
    M, N, K = 2 * bm, 3 * bn, steps * bk
    A, B = workloads.pair(M, N, K, "f16", "int", 820)
    C, _ = og.gemm(A, B, "f16")
    a, b = operands(A, B, "f16", layout)
    for P in (1, 4):
        s = ts.Schedule(order="grouped", group_m=2, mode="crosstile", num_programs=P, tile=tile)
        say(f"layout {layout} {M}x{N}x{K} {s.label()}")
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ts.gemm(a, b, out=c, schedule=s)
        torch.cuda.synchronize()
        bad = np.argwhere(to_f64(c) != C)
        assert bad.size == 0, f"{layout} P={P}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("tile", ["128x128x64", "256x256x64w8"])
@pytest.mark.parametrize("steps", [8, 9])
def test_nested_crosstile_padded_strides_with_canaries(layout, tile, steps):
    # the nested cross-tile kernel runs its slice offsets on by one row-stride-sized
    # step a K step: padded row strides of A, B and C (the operands inside larger
    # buffers, 16-byte aligned), exact integer products, and nothing written
    # outside C
    bm, bn, bk = (int(v) for v in tile[:-2 if tile[-2:] in ("w8", "pp") else None].split("x"))
    M, N, K = 2 * bm, 3 * bn, steps * bk
    A, B = workloads.pair(M, N, K, "f16", "int", 830)
    C, _ = og.gemm(A, B, "f16")
    pad = 24
    def padded(X, transposed):
        rows, cols = (X.shape[1], X.shape[0]) if transposed else X.shape
        buf = torch.zeros((rows, cols + pad), dtype=torch.float16, device="cuda")
        view = buf[:, :cols]
        view.copy_(to_device(np.ascontiguousarray(X.T) if transposed else X, "f16"))
        return view.t() if transposed else view
    a, b = padded(A, layout[0] == "T"), padded(B, layout[1] == "T")
    assert max(a.stride()) > (K if layout[0] == "N" else M) and max(b.stride()) > (N if layout[1] == "N" else K)
    assert ts.query(M, N, K, ts.Schedule(tile=tile))["masked"] == 0
    cbuf = torch.full((M + 4, N + 2 * pad), -12345.0, device="cuda")
    c = cbuf[2:2 + M, pad:pad + N]
    for P in (1, 4):
        c.fill_(float("nan"))
        s = ts.Schedule(order="grouped", group_m=2, mode="crosstile", num_programs=P, tile=tile)
        say(f"padded {layout} {M}x{N}x{K} {s.label()}")
        ts.gemm(a, b, out=c, schedule=s)
        torch.cuda.synchronize()
        bad = np.argwhere(to_f64(c) != C)
        assert bad.size == 0, f"{layout} P={P}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        guard = cbuf.clone()
        guard[2:2 + M, pad:pad + N] = -12345.0
        assert (guard == -12345.0).all(), "write outside C"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ab,c_dtype", [("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")])
def test_layouts_random_inputs_within_bound(layout, ab, c_dtype):
    M, N, K = 700, 900, 333
    A, B = workloads.pair(M, N, K, ab, "uniform" if ab == "f16" else "normal", 810)
    C, S = og.gemm(A, B, ab, threads=4)
    a, b = operands(A, B, ab, layout)
    s = ts.Schedule(order="auto", mode="auto")
    c = torch.empty((M, N), dtype=TORCH_OUT[c_dtype], device="cuda")
    say(f"layout {layout} {ab}->{c_dtype} {M}x{N}x{K}")
    ts.gemm(a, b, out=c, schedule=s)
    torch.cuda.synchronize()
    ok, worst, bad = og.accept(to_f64(c), C, S, c_dtype)
    assert ok, f"{layout}: {bad} outside the bound (worst {worst:.3g})"


@pytest.mark.parametrize("layout", ["NT", "TN", "TT"])
def test_transposed_headline_shape_sampled(layout):
    # 16384 x 16384 x 4096 with B stored [N][K] (the whole-tile path that stages B as A),
    # A stored [K][M] (A staged as B) or both
    w = workloads.SQ_16384
    A, B = workloads.inputs(w)
    a, b = operands(A, B, "f16", layout)
    out = {}
    for lay, (x, y) in ((layout, (a, b)), ("NN", (to_device(A, "f16"), to_device(B, "f16")))):
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        say(f"headline shape {lay}")
        ts.gemm(x, y, out=c, schedule=ts.Schedule(order="auto", mode="auto"))
        torch.cuda.synchronize()
        out[lay] = c
        del x, y
    # same tiles, same K order per element: bit-identical to the [M][K] x [K][N] layout
    assert torch.equal(out[layout], out["NN"])
    rng = np.random.default_rng(13)
    threads = max(1, min(16, og.max_threads()))
    for tm, tn in tile_sample(w.M, w.N, 256, 256, rng, n_random=16, groups=(8,)):
        r0, c0 = tm * 256, tn * 256
        C, S = og.gemm(A, B, "f16", rows=(r0, r0 + 256), cols=(c0, c0 + 256), threads=threads)
        ok, worst, bad = og.accept(to_f64(out[layout][r0:r0 + 256, c0:c0 + 256]), C, S, "f16")
        assert ok, f"tile ({tm}, {tn}): {bad} outside the bound"


def test_unsupported_strides_are_rejected():
    a = torch.zeros((64, 128), dtype=torch.float16, device="cuda")
    b = torch.zeros((128, 64), dtype=torch.float16, device="cuda")
    c = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    # neither stride of A is 1 (every other column of a wider matrix)
    wide = torch.zeros((64, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(ts.TsError) as e:
        ts.gemm(wide[:, ::2], b, out=c)
    assert e.value.status == ts.TS_ERR_UNSUPPORTED
    ts.gemm(a, b, out=c)
