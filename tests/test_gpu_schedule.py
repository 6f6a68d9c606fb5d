"""GPU schedule trace: the device computes each workgroup's (tile, K step)
sequence with the functions the GEMM kernels use; it must equal the oracle's
integer maps bit for bit."""
import numpy as np
import pytest
import torch

from oracle import schedule as osch
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_scheduling_amd as ts
else:
    ts = None


def _oracle(M, N, K, s, grid):
    q = ts.query(M, N, K, s)
    mode = {"tiled": osch.TILED, "persistent": osch.PERSISTENT, "crosstile": osch.CROSSTILE,
            "streamk": osch.STREAMK}[s.mode]
    order = osch.GROUPED if s.order == "grouped" else osch.ROW_MAJOR
    os_ = osch.Schedule(order=order, group_m=s.group_m, mode=mode, num_programs=grid,
                        xcd_remap=s.xcd_remap, xcds=q["xcds"])
    return osch.trace(M, N, K, q["block_m"], q["block_n"], q["block_k"], os_)


CASES = [(256, 256, 256, "64x64x32"), (5000, 12290, 1000, "256x256x64w8"), (8192, 8192, 4096, "256x256x64w8"),
         (16384, 16384, 128, "256x256x64w8"), (1000, 700, 0, "128x128x64"), (300, 520, 200, "64x64x32"),
         (5000, 12290, 1000, "256x256x64pp")]


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("order,G", [("row_major", 8), ("grouped", 4), ("grouped", 8), ("grouped", 16)])
@pytest.mark.parametrize("mode", ["tiled", "persistent", "crosstile", "streamk"])
@pytest.mark.parametrize("remap", [False, True])
def test_gpu_trace_equals_oracle(M, N, K, tile, order, G, mode, remap):
    s = ts.Schedule(order=order, group_m=G, mode=mode, num_programs=0, xcd_remap=remap, tile=tile)
    say(f"trace {M}x{N}x{K} {s.label()}")
    got = ts.schedule_trace(M, N, K, s).numpy()
    grid = ts.query(M, N, K, s)["grid"]
    ref = _oracle(M, N, K, s, grid)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_device_properties_and_auto_grid():
    q = ts.query(16384, 16384, 4096, ts.Schedule(mode="persistent"))
    say(f"query {q}")
    assert q["cu_count"] > 0 and q["programs_per_cu"] >= 1
    assert q["grid"] == min(q["cu_count"] * q["programs_per_cu"], q["num_tiles"])
    assert q["scratch_bytes"] >= 0 and q["vgprs"] > 0


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("mode", ["tiled", "persistent", "auto"])
def test_gpu_auto_order_is_the_models_choice(M, N, K, tile, mode):
    from oracle import model as om

    s = ts.Schedule(order="auto", mode=mode, tile=tile)
    q = ts.query(M, N, K, s)
    concurrent = min(q["cu_count"] * q["programs_per_cu"], q["grid"])
    order, G, remap, pm = om.choose_order(q["num_m_tiles"], q["num_n_tiles"], q["grid"], concurrent, q["xcds"])
    got = ("grouped" if q["order"] == 1 else "row_major", q["group_m"] if q["order"] == 1 else 1, bool(q["xcd_remap"]))
    say(f"auto order {M}x{N}x{K} {tile} {mode}: {got}, model reuse {q['model_l2_reuse_pm']}")
    assert got == (order, G, remap) and q["model_l2_reuse_pm"] == pm
    resolved_mode = {0: "tiled", 1: "persistent", 2: "crosstile"}[q["mode"]]
    resolved = ts.Schedule(order=order, group_m=G, mode=resolved_mode, xcd_remap=remap, tile=tile)
    got_tr = ts.schedule_trace(M, N, K, s).numpy()
    ref = _oracle(M, N, K, resolved, q["grid"])
    assert np.array_equal(got_tr, ref)


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("mode", ["persistent", "crosstile", "streamk"])
def test_gpu_trace_mulshift_equals_oracle(M, N, K, tile, mode):
    s = ts.Schedule(order="grouped", group_m=8, mode=mode, xcd_remap=True, tile=tile, index_math="mulshift")
    got = ts.schedule_trace(M, N, K, s).numpy()
    ref = _oracle(M, N, K, s, ts.query(M, N, K, s)["grid"])
    assert np.array_equal(got, ref)
