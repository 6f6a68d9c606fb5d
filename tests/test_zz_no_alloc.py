"""ts_gemm_noalloc: the stream-K launch without a caller workspace (the library's
static per-GPU scratch array) gives the same C as ts_gemm_workspace with a
caller-owned workspace, on two calls in a row, the second with a smaller input,
and stays within the oracle's bound."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from tests.gpu_helpers import say, to_device, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_scheduling_amd as ts
else:
    ts = None


def _call(fn, a, b, c, sched, ab, ct, *ws):
    M, K = a.shape
    N = b.shape[1]
    st = fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, a.stride(0), 1, b.stride(0), 1, c.stride(0), 1,
            ab, ct, ctypes.byref(sched._c()), torch.cuda.current_stream().cuda_stream, *ws)
    assert st == ts.TS_OK, ts.status_string(st)


@pytest.mark.parametrize("shapes", [((5000, 12290, 1000), (1000, 2000, 300)),
                                    ((1500, 1800, 700), (333, 290, 150))])
def test_noalloc_equals_workspace_entry_point(shapes):
    sched = ts.Schedule(order="grouped", group_m=8, mode="streamk", xcd_remap=True)
    for i, (M, N, K) in enumerate(shapes):
        A, B = workloads.pair(M, N, K, "bf16", "normal", 700 + i)
        a, b = to_device(A, "bf16"), to_device(B, "bf16")
        q = ts.query(M, N, K, sched, ts.TS_BF16, ts.TS_F32)
        assert 0 < q["workspace_bytes"] <= ts._lib.ts_noalloc_scratch_bytes()
        ws = torch.zeros(q["workspace_bytes"], dtype=torch.uint8, device="cuda")
        c_ws = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        c_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        say(f"noalloc call {i}: {M}x{N}x{K} {sched.label()} workspace {q['workspace_bytes']}")
        _call(ts._lib.ts_gemm_workspace, a, b, c_ws, sched, ts.TS_BF16, ts.TS_F32, ws.data_ptr(), ws.numel())
        _call(ts._lib.ts_gemm_noalloc, a, b, c_na, sched, ts.TS_BF16, ts.TS_F32)
        torch.cuda.synchronize()
        assert torch.equal(c_ws, c_na), f"call {i}"
        # a sample of rows against the oracle (the split tiles sit in the last rows)
        rows = sorted({0, M // 2, M - 1, M - 2, M - 257})
        for r in rows:
            C, S = og.gemm(A, B, "bf16", rows=(r, r + 1), threads=8)
            ok, worst, bad = og.accept(to_f64(c_na[r:r + 1]), C, S, "f32")
            assert ok, f"call {i} row {r}: {bad} outside the bound (worst {worst:.3g})"


def test_noalloc_without_split_is_ts_gemm():
    M, N, K = 1024, 1536, 512
    A, B = workloads.pair(M, N, K, "f16", "uniform", 710)
    a, b = to_device(A, "f16"), to_device(B, "f16")
    for mode in ("tiled", "persistent", "crosstile"):
        sched = ts.Schedule(order="grouped", group_m=4, mode=mode, xcd_remap=True)
        c1 = torch.empty((M, N), dtype=torch.float16, device="cuda")
        c2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
        _call(ts._lib.ts_gemm, a, b, c1, sched, ts.TS_F16, ts.TS_F16)
        _call(ts._lib.ts_gemm_noalloc, a, b, c2, sched, ts.TS_F16, ts.TS_F16)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2), mode


def test_noalloc_rejects_launches_beyond_the_scratch_array():
    # 64 x 64 tiles of 16 KiB each: 8192 programs need 128 MiB of partial tiles
    sched = ts.Schedule(mode="streamk", num_programs=8191, tile="64x64x32")
    q = ts.query(4096, 4096, 512, sched)
    assert q["workspace_bytes"] > ts._lib.ts_noalloc_scratch_bytes()
    a = torch.zeros((4096, 512), dtype=torch.float16, device="cuda")
    b = torch.zeros((512, 4096), dtype=torch.float16, device="cuda")
    c = torch.zeros((4096, 4096), dtype=torch.float16, device="cuda")
    st = ts._lib.ts_gemm_noalloc(a.data_ptr(), b.data_ptr(), c.data_ptr(), 4096, 4096, 512, 512, 1, 4096, 1,
                                 4096, 1, ts.TS_F16, ts.TS_F16, ctypes.byref(sched._c()), None)
    assert st == ts.TS_ERR_UNSUPPORTED
