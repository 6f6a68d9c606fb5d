"""The C-ABI library on the CPU: loads, exports every declared symbol, validates
arguments before any HIP call, and its host-side schedule equals the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import tile_scheduling_amd as ts
from oracle import schedule as osch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "tsgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert set(names) == set(ts.EXPORTS)
    lib = ctypes.CDLL(ts.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert ts.status_string(code).startswith("TS_")
    assert "unknown" in ts.status_string(17)


# ---- validation happens before any HIP call (fake pointers are never touched) ------

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below is rejected first


@pytest.mark.parametrize("kw,expect", [
    (dict(M=-1), ts.TS_ERR_INVALID_ARG),
    (dict(K=-5), ts.TS_ERR_INVALID_ARG),
    (dict(ab=ts.TS_F16, c=ts.TS_BF16), ts.TS_ERR_UNSUPPORTED),
    (dict(ab=ts.TS_F32, c=ts.TS_F32), ts.TS_ERR_UNSUPPORTED),
    (dict(ab=9), ts.TS_ERR_INVALID_ARG),
    (dict(strides=(64, 2, 64, 1, 64, 1)), ts.TS_ERR_UNSUPPORTED),      # neither A stride is 1
    (dict(strides=(64, 1, 64, 2, 64, 1)), ts.TS_ERR_UNSUPPORTED),      # neither B stride is 1
    (dict(strides=(1, 10, 64, 1, 64, 1)), ts.TS_ERR_INVALID_ARG),      # A stored [K][M] with stride < M
    (dict(strides=(64, 1, 1, 10, 64, 1)), ts.TS_ERR_INVALID_ARG),      # B stored [N][K] with stride < K
    (dict(strides=(64, 1, 64, 1, 64, 3)), ts.TS_ERR_UNSUPPORTED),
    (dict(strides=(10, 1, 64, 1, 64, 1)), ts.TS_ERR_INVALID_ARG),   # lda < K
    (dict(strides=(64, 1, 64, 1, 10, 1)), ts.TS_ERR_INVALID_ARG),   # ldc < N
    (dict(a=FAKE + 1), ts.TS_ERR_ALIGNMENT),
    (dict(c=ts.TS_F32, cptr=FAKE + 2), ts.TS_ERR_ALIGNMENT),
    (dict(cptr=0), ts.TS_ERR_INVALID_ARG),
    (dict(a=0), ts.TS_ERR_INVALID_ARG),
    (dict(sched=ts.Schedule(order="grouped", group_m=0)), ts.TS_ERR_INVALID_ARG),
    (dict(sched=ts.Schedule(mode="persistent", num_programs=-3)), ts.TS_ERR_INVALID_ARG),
])
def test_invalid_arguments_are_rejected(kw, expect):
    M, N, K = kw.get("M", 64), 64, kw.get("K", 64)
    st = ts.gemm_raw(kw.get("a", FAKE), FAKE, kw.get("cptr", FAKE), M, N, K,
                     strides=kw.get("strides", (64, 1, 64, 1, 64, 1)),
                     ab_dtype=kw.get("ab", ts.TS_F16), c_dtype=kw.get("c", ts.TS_F16),
                     schedule=kw.get("sched"))
    assert st == expect, ts.status_string(st)


def test_bad_schedule_enums_are_rejected():
    s = ts._Schedule(5, 1, 0, 0, 0, 0)
    assert ts._lib.ts_gemm(FAKE, FAKE, FAKE, 64, 64, 64, 64, 1, 64, 1, 64, 1, 1, 1, ctypes.byref(s), None) == -1
    for bad in (ts._Schedule(0, 1, 5, 0, 0, 0), ts._Schedule(0, 1, 0, 0, 2, 0), ts._Schedule(0, 1, 0, 0, 0, 6),
                ts._Schedule(3, 1, 0, 0, 0, 0), ts._Schedule(0, 1, 0, 0, 0, 0, 2)):
        assert ts._lib.ts_gemm(FAKE, FAKE, FAKE, 64, 64, 64, 64, 1, 64, 1, 64, 1, 1, 1, ctypes.byref(bad), None) == -1


def test_empty_output_is_a_no_op():
    assert ts.gemm_raw(0, 0, 0, 0, 64, 64) == ts.TS_OK
    assert ts.gemm_raw(0, 0, 0, 64, 0, 64) == ts.TS_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_gpu_reports_no_device():
    assert ts.gemm_raw(FAKE, FAKE, FAKE, 64, 64, 64) == ts.TS_ERR_NO_DEVICE


# ---- launch planning ---------------------------------------------------------------

def test_query_tile_grid_and_masking():
    q = ts.query(256, 256, 256, ts.Schedule(tile="64x64x32"), ts.TS_F16, ts.TS_F32)
    assert (q["block_m"], q["block_n"], q["block_k"]) == (64, 64, 32)
    assert (q["num_m_tiles"], q["num_n_tiles"], q["k_steps"], q["grid"], q["masked"]) == (4, 4, 8, 16, 0)
    q = ts.query(5000, 12290, 1000, ts.Schedule(mode="persistent", num_programs=256, tile="256x256x64"),
                 ts.TS_BF16, ts.TS_F32)
    assert (q["num_m_tiles"], q["num_n_tiles"], q["k_steps"]) == (20, 49, 16)
    assert q["grid"] == 256 and q["masked"] == 2   # edge path (B rows only 4-byte aligned)
    # kernel path: whole tiles 0, masked registers 1, zero-filled edges 2
    assert ts.query(1000, 1024, 512, ts.Schedule(tile="256x256x64"))["masked"] == 2
    assert ts.query(1000, 1025, 512, ts.Schedule(tile="256x256x64"))["masked"] == 1   # N odd
    assert ts.query(1000, 1024, 500, ts.Schedule(tile="256x256x64"))["masked"] == 1   # K not 0 mod 8
    assert ts.query(1000, 1024, 512, ts.Schedule(tile="64x64x32"))["masked"] == 1     # no direct-to-LDS tile
    q = ts.query(16384, 16384, 4096, ts.Schedule())
    assert (q["block_m"], q["num_tiles"], q["masked"]) == (256, 4096, 0)
    # rows too long for 32-bit in-tile offsets of the unmasked kernels: masked path
    assert ts.query(256, 256, 1 << 22, ts.Schedule(tile="256x256x64"))["masked"] == 1
    assert ts.query(256, 1 << 25, 64, ts.Schedule(tile="256x256x64"))["masked"] == 1
    assert ts.query(256, 256, 1 << 21, ts.Schedule(tile="256x256x64"))["masked"] == 0
    q = ts.query(64, 64, 0, ts.Schedule(mode="crosstile", num_programs=8))
    assert q["k_steps"] == 0 and q["masked"] == 1  # K = 0 still writes C (zeros)


def test_pingpong_tile_has_the_8_wave_tiles_geometry():
    # same tile, threads and LDS as the 8-wave configuration; stream-K and the masked
    # register path run the 8-wave kernels
    for M, N, K, mode in [(16384, 16384, 4096, "persistent"), (5000, 12290, 1000, "crosstile"),
                          (1000, 1001, 77, "persistent"), (5000, 12290, 1000, "streamk")]:
        qs = [ts.query(M, N, K, ts.Schedule(order="grouped", group_m=8, mode=mode, num_programs=256, tile=t))
              for t in ("256x256x64w8", "256x256x64pp")]
        for key in ("block_m", "block_n", "block_k", "grid", "threads", "lds_bytes", "masked", "workspace_bytes"):
            assert qs[0][key] == qs[1][key], key


def test_four_wave_256_tile_has_no_crosstile_kernel():
    s = ts.Schedule(mode="crosstile", num_programs=8, tile="256x256x64")
    with pytest.raises(ts.TsError) as e:
        ts.query(1024, 1024, 512, s)
    assert e.value.status == ts.TS_ERR_UNSUPPORTED
    assert ts.gemm_raw(FAKE, FAKE, FAKE, 1024, 1024, 512, schedule=s) == ts.TS_ERR_UNSUPPORTED
    for mode in ("tiled", "persistent"):
        ts.query(1024, 1024, 512, ts.Schedule(mode=mode, num_programs=8, tile="256x256x64"))


@pytest.mark.parametrize("tile", ["64x64x32", "128x128x64", "256x256x64", "256x256x64w8", "256x256x64pp"])
@pytest.mark.parametrize("M,N,K", [(16384, 16384, 4096), (5000, 12290, 1000), (333, 290, 150)])
@pytest.mark.parametrize("mode", ["tiled", "persistent", "crosstile"])
def test_query_reports_the_compilers_resource_use(tile, M, N, K, mode):
    if tile == "256x256x64" and mode == "crosstile":
        return
    q = ts.query(M, N, K, ts.Schedule(mode=mode, num_programs=8, tile=tile))
    # recorded at build time for every kernel instance: no device needed
    assert q["arch_vgprs"] > 0 and q["agprs"] >= 0 and q["sgprs"] > 0, q
    assert q["arch_vgprs"] + q["agprs"] <= 512
    assert q["spilled_vgprs"] >= 0 and q["spilled_sgprs"] >= 0
    assert q["compiler_occupancy"] >= 1
    threads = q["threads"]
    # one workgroup's waves must fit one CU's register file (4 SIMDs x 512 registers per lane)
    waves_per_simd = -(-threads // 64 // 4)
    assert waves_per_simd * (q["arch_vgprs"] + q["agprs"]) <= 512


@pytest.mark.parametrize("M,K,kind", [(16384, 64, "flat"), (16384, 128, "plain"), (16384, 192, "plain"),
                                      (16384, 448, "plain"), (16384, 512, "plain"), (16384, 576, "plain"),
                                      (16384, 4096, "plain"), (16384, 4160, "plain"), (4096, 256, "flat"),
                                      (4096, 512, "deferred"), (4096, 4096, "deferred")])
def test_crosstile_kernel_choice_by_k_steps(M, K, kind):
    # the cross-tile mode on the 8-wave tile runs the nested kernel without the
    # deferred wait when a program has more than one tile (16384^2 on 256 programs:
    # 16) and at least 2 K steps; with one tile per program (4096^2: 256 tiles) the
    # nested kernel with the deferred wait from 8 K steps on; the flattened loop
    # otherwise (one K step; one tile of 2 to 7).  The resource report follows the
    # kernel that runs, and the nested kernels spill no vector registers.
    s = ts.Schedule(order="grouped", group_m=8, xcd_remap=True, mode="crosstile", num_programs=256,
                    tile="256x256x64w8")
    report = lambda x: (x["arch_vgprs"], x["spilled_vgprs"], x["sgprs"], x["spilled_sgprs"])
    ref = {"plain": ts.query(16384, 16384, 512, s), "deferred": ts.query(4096, 4096, 4096, s),
           "flat": ts.query(16384, 16384, 64, s)}
    assert len({report(r) for r in ref.values()}) == 3, ref   # three kernels, told apart by their reports
    q = ts.query(M, M, K, s)
    assert q["mode"] == 2
    assert report(q) == report(ref[kind]), (kind, q)
    if kind != "flat":
        assert q["spilled_vgprs"] == 0, q
    # the automatic schedule of the headline shape resolves to a nested kernel
    if K == 4096 and M == 16384:
        qa = ts.query(16384, 16384, K, ts.Schedule(order="auto", mode="auto", num_programs=256))
        assert qa["mode"] == 2 and report(qa) == report(ref["plain"])


# ---- host-side schedule (the same functions the kernels run) vs the oracle ----------

def _oracle_sched(s: ts.Schedule, grid_programs):
    mode = {"tiled": osch.TILED, "persistent": osch.PERSISTENT, "crosstile": osch.CROSSTILE,
            "streamk": osch.STREAMK}[s.mode]
    order = osch.GROUPED if s.order == "grouped" else osch.ROW_MAJOR
    return osch.Schedule(order=order, group_m=s.group_m, mode=mode, num_programs=grid_programs,
                         xcd_remap=s.xcd_remap)


CASES = [
    (256, 256, 256, "64x64x32"),
    (300, 520, 200, "64x64x32"),
    (1000, 700, 96, "128x128x64"),
    (5000, 12290, 1000, "256x256x64w8"),
    (2048, 3072, 0, "256x256x64w8"),
    (64, 64, 33, "64x64x32"),
    (5000, 12290, 1000, "256x256x64pp"),
]


@pytest.mark.parametrize("M,N,K,tile", CASES)
@pytest.mark.parametrize("order,G", [("row_major", 1), ("grouped", 3), ("grouped", 8), ("grouped", 100)])
@pytest.mark.parametrize("mode,P", [("tiled", 0), ("persistent", 7), ("persistent", 256), ("crosstile", 256),
                                    ("streamk", 7), ("streamk", 256)])
@pytest.mark.parametrize("remap", [False, True])
def test_host_trace_equals_oracle(M, N, K, tile, order, G, mode, P, remap):
    s = ts.Schedule(order=order, group_m=G, mode=mode, num_programs=P, xcd_remap=remap, tile=tile)
    got = ts.schedule_trace_host(M, N, K, s)
    bm, bn, bk = (int(v) for v in tile.replace("w8", "").replace("pp", "").split("x"))
    ref = osch.trace(M, N, K, bm, bn, bk, _oracle_sched(s, P))
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_host_trace_auto_grid_uses_cus_times_occupancy():
    s = ts.Schedule(order="grouped", group_m=8, mode="persistent", tile="256x256x64")
    got = ts.schedule_trace_host(8192, 8192, 4096, s, cu_count=256, programs_per_cu=1)
    ref = osch.trace(8192, 8192, 4096, 256, 256, 64, _oracle_sched(s, 256))
    assert np.array_equal(got, ref)
    with pytest.raises(ts.TsError):
        ts.schedule_trace_host(8192, 8192, 4096, s)  # no device and no CU count given


@pytest.mark.parametrize("M,N,K,tile,P", [(5000, 12290, 1000, "256x256x64w8", 256), (300, 520, 200, "64x64x32", 7),
                                         (1000, 700, 96, "128x128x64", 512), (512, 512, 0, "128x128x64", 5),
                                         (8192, 8192, 4096, "256x256x64w8", 256)])
def test_streamk_workspace_size(M, N, K, tile, P):
    q = ts.query(M, N, K, ts.Schedule(mode="streamk", num_programs=P, tile=tile))
    T, ks, grid = q["num_tiles"], q["k_steps"], q["grid"]
    assert grid == min(P, T * max(ks, 1))
    split = T % grid if ks > 0 else 0
    if split == 0:
        assert q["workspace_bytes"] == 0
    else:
        header = -(-(grid + 1) * 4 // 256) * 256
        assert q["workspace_bytes"] == header + grid * q["block_m"] * q["block_n"] * 4
    for mode in ("tiled", "persistent", "crosstile"):
        assert ts.query(M, N, K, ts.Schedule(mode=mode, num_programs=P, tile=tile))["workspace_bytes"] == 0


def test_streamk_needs_its_workspace():
    s = ts.Schedule(mode="streamk", num_programs=256, tile="256x256x64w8")
    need = ts.query(5000, 12290, 1000, s, ts.TS_BF16, ts.TS_F32)["workspace_bytes"]
    assert need > 0
    args = [FAKE, FAKE, FAKE, 5000, 12290, 1000, 1000, 1, 12290, 1, 12290, 1, ts.TS_BF16, ts.TS_F32,
            ctypes.byref(s._c()), None]
    # without a workspace, too small, or misaligned: rejected before any HIP call
    assert ts._lib.ts_gemm(*args) == ts.TS_ERR_INVALID_ARG
    assert ts._lib.ts_gemm_workspace(*args, None, 0) == ts.TS_ERR_INVALID_ARG
    assert ts._lib.ts_gemm_workspace(*args, FAKE, need - 1) == ts.TS_ERR_INVALID_ARG
    assert ts._lib.ts_gemm_workspace(*args, FAKE + 16, need) == ts.TS_ERR_INVALID_ARG
    assert ts._lib.ts_gemm_workspace(*args, FAKE, -1) == ts.TS_ERR_INVALID_ARG


def test_noalloc_refuses_oversize_launches_before_any_hip_call():
    cap = ts._lib.ts_noalloc_scratch_bytes()
    assert cap == (64 << 20) + (64 << 10)
    big = ts.Schedule(mode="streamk", num_programs=8191, tile="64x64x32")
    assert ts.query(4096, 4096, 512, big)["workspace_bytes"] > cap
    assert ts._lib.ts_gemm_noalloc(FAKE, FAKE, FAKE, 4096, 4096, 512, 512, 1, 4096, 1, 4096, 1, ts.TS_F16,
                                   ts.TS_F16, ctypes.byref(big._c()), None) == ts.TS_ERR_UNSUPPORTED
    small = ts.Schedule(mode="streamk", num_programs=256, tile="256x256x64w8")
    assert 0 < ts.query(5000, 12290, 1000, small, ts.TS_BF16, ts.TS_F32)["workspace_bytes"] <= cap


# ---- per-shape schedule choice (TS_ORDER_AUTO, TS_MODE_AUTO) ---------------------------

@pytest.mark.parametrize("M,N,K,tile,mode,P", [
    (16384, 16384, 4096, "256x256x64w8", "persistent", 256), (8192, 8192, 4096, "256x256x64w8", "persistent", 256),
    (5000, 12290, 1000, "256x256x64w8", "tiled", 0), (5000, 12290, 1000, "256x256x64w8", "persistent", 256),
    (16384, 16384, 4096, "128x128x64", "persistent", 512), (2048, 16384, 4096, "256x256x64w8", "tiled", 0),
    (4096, 4096, 4096, "128x128x64", "tiled", 0), (1000, 64000, 512, "128x128x64", "persistent", 300),
    (3000, 700, 256, "64x64x32", "tiled", 0)])
def test_auto_order_is_the_models_choice(M, N, K, tile, mode, P):
    from oracle import model as om

    q = ts.query(M, N, K, ts.Schedule(order="auto", mode=mode, num_programs=P, tile=tile))
    # without a device the library takes 256 resident workgroups
    concurrent = min(256, q["grid"])
    order, G, remap, pm = om.choose_order(q["num_m_tiles"], q["num_n_tiles"], q["grid"], concurrent, 8)
    got = ("grouped" if q["order"] == 1 else "row_major", q["group_m"] if q["order"] == 1 else 1,
           bool(q["xcd_remap"]))
    assert got == (order, G, remap)
    assert q["model_l2_reuse_pm"] == pm
    # the trace of the resolved schedule equals the oracle's for it
    sched = ts.Schedule(order=order, group_m=G, mode=mode, num_programs=P, xcd_remap=remap, tile=tile)
    auto = ts.Schedule(order="auto", mode=mode, num_programs=P, tile=tile)
    if q["grid"] * q["trace_items"] <= 300000:
        assert np.array_equal(ts.schedule_trace_host(M, N, K, auto), ts.schedule_trace_host(M, N, K, sched))


@pytest.mark.parametrize("K,expect", [(128, "crosstile"), (1024, "crosstile"), (1025, "crosstile"),
                                      (2048, "crosstile"), (2049, "crosstile"), (4096, "crosstile"),
                                      (4160, "crosstile"), (8192, "crosstile"), (0, "crosstile")])
def test_auto_mode_by_k_steps(K, expect):
    # the 8-wave tile: the flattened loop up to 32 K steps, the nested cross-tile
    # kernel from 8 steps on, so cross-tile at every K
    q = ts.query(16384, 16384, K, ts.Schedule(order="auto", mode="auto", num_programs=256, tile="256x256x64w8"))
    assert q["mode"] == {"persistent": 1, "crosstile": 2}[expect]
    # the 64 x 64 tile has no nested kernel: persistent above 32 K steps
    q = ts.query(16384, 16384, K, ts.Schedule(mode="auto", num_programs=256, tile="64x64x32"))
    assert q["mode"] == (2 if -(-K // 32) <= 32 else 1)
    # the 4-wave 256 tile has no cross-tile kernel: auto falls back to persistent
    q = ts.query(16384, 16384, 128, ts.Schedule(mode="auto", num_programs=256, tile="256x256x64"))
    assert q["mode"] == 1


@pytest.mark.parametrize("order,G", [("row_major", 1), ("grouped", 3), ("grouped", 8), ("grouped", 100)])
@pytest.mark.parametrize("M,N", [(5000, 12290), (16384, 16384), (333, 290), (70000, 300)])
def test_mulshift_index_math_gives_the_same_map(order, G, M, N):
    for mode, P in (("persistent", 256), ("crosstile", 7), ("tiled", 0), ("streamk", 256)):
        a = ts.Schedule(order=order, group_m=G, mode=mode, num_programs=P, xcd_remap=True, tile="128x128x64")
        b = ts.Schedule(order=order, group_m=G, mode=mode, num_programs=P, xcd_remap=True, tile="128x128x64",
                        index_math="mulshift")
        assert ts.query(M, N, 256, b)["index_math"] == 1
        assert np.array_equal(ts.schedule_trace_host(M, N, 256, a), ts.schedule_trace_host(M, N, 256, b))


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
@pytest.mark.parametrize("strides", [(64, 1, 64, 1, 64, 1), (64, 1, 1, 64, 64, 1), (1, 64, 64, 1, 64, 1),
                                     (1, 64, 1, 64, 64, 1)], ids=["NN", "NT", "TN", "TT"])
def test_four_layouts_pass_validation(strides):
    # valid: rejected only because there is no device
    assert ts.gemm_raw(FAKE, FAKE, FAKE, 64, 64, 64, strides=strides) == ts.TS_ERR_NO_DEVICE

def test_phase_probe_validates_before_any_hip_call():
    sink = ctypes.c_float(0.0)
    flops = ctypes.c_double(0.0)
    for iters, pattern in ((0, 0), (10, -1), (10, 4)):
        assert ts._lib.ts_mfma_phase_probe(iters, pattern, ctypes.addressof(sink), 1 << 20, ctypes.byref(flops),
                                           None) == ts.TS_ERR_INVALID_ARG
    assert ts._lib.ts_mfma_phase_probe(10, 2, None, 1 << 20, ctypes.byref(flops), None) == ts.TS_ERR_INVALID_ARG
