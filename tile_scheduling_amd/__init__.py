"""Python binding of libtsgemm (tiled GEMM with tile-order schedules, MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libtsgemm.so``.  PyTorch supplies device memory and streams.  The
library is built in-tree by ``python -m tile_scheduling_amd.build``; importing
this package without it raises ImportError, and there is no fallback path.

    import torch, tile_scheduling_amd as ts
    c = ts.gemm(a, b, out_dtype=torch.float16,
                schedule=ts.Schedule(order="grouped", group_m=8, mode="persistent"))
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch  # loaded first: libtsgemm binds to the HIP runtime torch already loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tile_scheduling_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

# status codes, element types and schedule enums (include/tsgemm.h)
TS_OK, TS_ERR_INVALID_ARG, TS_ERR_UNSUPPORTED, TS_ERR_ALIGNMENT, TS_ERR_HIP, TS_ERR_NO_DEVICE = 0, -1, -2, -3, -4, -5
TS_F16, TS_BF16, TS_F32 = 1, 2, 3
ORDERS = {"row_major": 0, "grouped": 1, "auto": 2}
MODES = {"tiled": 0, "persistent": 1, "crosstile": 2, "streamk": 3, "auto": 4}
INDEX_MATH = {"divide": 0, "mulshift": 1}
TILES = {"auto": 0, "64x64x32": 1, "128x128x64": 2, "256x256x64": 3, "256x256x64w8": 4, "256x256x64pp": 5}


class _Schedule(ctypes.Structure):
    _fields_ = [("order", _i32), ("group_m", _i32), ("mode", _i32),
                ("num_programs", _i32), ("xcd_remap", _i32), ("tile_config", _i32), ("index_math", _i32)]


class LaunchInfo(ctypes.Structure):
    _fields_ = [("block_m", _i32), ("block_n", _i32), ("block_k", _i32), ("threads", _i32),
                ("num_m_tiles", _i64), ("num_n_tiles", _i64), ("k_steps", _i64), ("num_tiles", _i64),
                ("grid", _i64), ("programs_per_cu", _i32), ("cu_count", _i32), ("xcds", _i32),
                ("lds_bytes", _i32), ("masked", _i32), ("workspace_bytes", _i64), ("trace_items", _i64),
                ("vgprs", _i32), ("scratch_bytes", _i32),
                ("arch_vgprs", _i32), ("agprs", _i32), ("sgprs", _i32), ("spilled_vgprs", _i32),
                ("spilled_sgprs", _i32), ("compiler_occupancy", _i32),
                ("order", _i32), ("group_m", _i32), ("mode", _i32), ("xcd_remap", _i32), ("index_math", _i32),
                ("model_l2_reuse_pm", _i32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib.ts_gemm.argtypes = [_p, _p, _p] + [_i64] * 9 + [_i32, _i32, ctypes.POINTER(_Schedule), _p]
_lib.ts_gemm.restype = _i32
_lib.ts_gemm_workspace.argtypes = _lib.ts_gemm.argtypes + [_p, _i64]
_lib.ts_gemm_workspace.restype = _i32
_lib.ts_gemm_noalloc.argtypes = list(_lib.ts_gemm.argtypes)
_lib.ts_gemm_noalloc.restype = _i32
_lib.ts_noalloc_scratch_bytes.argtypes = []
_lib.ts_noalloc_scratch_bytes.restype = _i64
_lib.ts_gemm_clocked.argtypes = _lib.ts_gemm.argtypes + [_p, _i64, _p, _i64]
_lib.ts_gemm_clocked.restype = _i32
_lib.ts_mfma_loop_probe.argtypes = [_i32, _p, _i64, ctypes.POINTER(ctypes.c_double), _p]
_lib.ts_mfma_loop_probe.restype = _i32
_lib.ts_mfma_phase_probe.argtypes = [_i32, _i32, _p, _i64, ctypes.POINTER(ctypes.c_double), _p]
_lib.ts_mfma_phase_probe.restype = _i32
_lib.ts_schedule_trace.argtypes = [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_Schedule), _p, _i64, _p]
_lib.ts_schedule_trace.restype = _i32
_lib.ts_schedule_trace_host.argtypes = [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_Schedule),
                                        _i32, _i32, _p, _i64]
_lib.ts_schedule_trace_host.restype = _i32
_lib.ts_query.argtypes = [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_Schedule), ctypes.POINTER(LaunchInfo)]
_lib.ts_query.restype = _i32
_lib.ts_status_string.argtypes = [_i32]
_lib.ts_status_string.restype = ctypes.c_char_p

EXPORTS = ("ts_gemm", "ts_gemm_workspace", "ts_gemm_noalloc", "ts_noalloc_scratch_bytes", "ts_gemm_clocked", "ts_schedule_trace", "ts_schedule_trace_host", "ts_query",
           "ts_status_string", "ts_mfma_loop_probe", "ts_mfma_phase_probe")


class TsError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(status_string(status))


def status_string(status: int) -> str:
    return _lib.ts_status_string(int(status)).decode()


@dataclasses.dataclass(frozen=True)
class Schedule:
    """Tile order and mode of one launch (see ts_schedule in include/tsgemm.h)."""

    order: str = "row_major"      # "row_major" | "grouped" | "auto"
    group_m: int = 8              # GROUP_SIZE_M for the grouped order
    mode: str = "tiled"           # "tiled" | "persistent" | "crosstile" | "streamk" | "auto"
    num_programs: int = 0         # persistent grid; 0 = CUs x workgroups per CU
    xcd_remap: bool = False       # contiguous tile-id runs per XCD
    tile: str = "auto"            # "auto" | "64x64x32" | "128x128x64" | "256x256x64" | "256x256x64w8" | "256x256x64pp"
    index_math: str = "divide"    # "divide" | "mulshift"

    def _c(self) -> _Schedule:
        return _Schedule(ORDERS[self.order], int(self.group_m), MODES[self.mode],
                         int(self.num_programs), 1 if self.xcd_remap else 0, TILES[self.tile],
                         INDEX_MATH[self.index_math])

    def label(self) -> str:
        o = {"row_major": "rowmajor", "auto": "autoorder"}.get(self.order, f"grouped{self.group_m}")
        r = "+remap" if self.xcd_remap and self.order != "auto" else ""
        p = f"/P{self.num_programs}" if self.mode != "tiled" and self.num_programs else ""
        x = "/mulshift" if self.index_math == "mulshift" else ""
        return f"{o}{r}/{self.mode}{p}/{self.tile}{x}"


_TORCH_DTYPE = {torch.float16: TS_F16, torch.bfloat16: TS_BF16, torch.float32: TS_F32}


def _check(status: int):
    if status != TS_OK:
        raise TsError(status)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_WORKSPACES: dict = {}


def workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A zeroed device workspace of at least ``nbytes`` for ts_gemm_workspace, one per
    device and stream, reused by later calls (every call leaves its flags zero)."""
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def gemm(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
         out_dtype: torch.dtype | None = None, schedule: Schedule | None = None,
         ws: torch.Tensor | None = None) -> torch.Tensor:
    """C = A @ B with A [M,K], B [K,N] fp16/bf16 CUDA tensors; C fp16/bf16/fp32.

    Enqueued on the current stream of A's device; returns C (``out`` if given).
    A stream-K schedule that splits tiles runs with ``ws`` (a uint8 CUDA tensor
    of at least ``query(...)["workspace_bytes"]`` bytes whose header is zero), or
    with a cached zeroed workspace of the device and stream.
    """
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {tuple(a.shape)} @ {tuple(b.shape)} do not multiply")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("A and B must be on the same GPU")
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or a.dtype, device=a.device)
    elif out.shape != (M, N) or out.device != a.device:
        raise ValueError("out has the wrong shape or device")
    sched = schedule or Schedule()
    s = sched._c()
    ab_t, c_t = _TORCH_DTYPE.get(a.dtype, 0), _TORCH_DTYPE.get(out.dtype, 0)
    if sched.mode == "streamk":
        need = query(M, N, K, sched, ab_t, c_t)["workspace_bytes"]
        if ws is None and need > 0:
            ws = workspace(need, a.device)
        wptr, wbytes = (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
        st = _lib.ts_gemm_workspace(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                                    a.stride(0), a.stride(1), b.stride(0), b.stride(1), out.stride(0),
                                    out.stride(1), ab_t, c_t, ctypes.byref(s), _stream_handle(a.device),
                                    wptr, wbytes)
    else:
        st = _lib.ts_gemm(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                          a.stride(0), a.stride(1), b.stride(0), b.stride(1), out.stride(0), out.stride(1),
                          ab_t, c_t, ctypes.byref(s), _stream_handle(a.device))
    _check(st)
    return out


def gemm_clocked(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor, schedule: Schedule | None = None):
    """ts_gemm_clocked: C = A @ B into ``out`` plus the per-workgroup clock record.

    Returns an int64 [grid, 4] CUDA tensor (shader-clock counter at start and end,
    100 MHz counter at start and end of every workgroup); use ``clock_ghz`` on it.
    """
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0] or out.shape != (a.shape[0], b.shape[1]):
        raise ValueError("shapes do not multiply")
    M, K = a.shape
    N = b.shape[1]
    sched = schedule or Schedule()
    grid = query(M, N, K, sched, _TORCH_DTYPE.get(a.dtype, 0), _TORCH_DTYPE.get(out.dtype, 0))["grid"]
    rec = torch.zeros((max(grid, 1), 4), dtype=torch.int64, device=a.device)
    s = sched._c()
    ab_t, c_t = _TORCH_DTYPE.get(a.dtype, 0), _TORCH_DTYPE.get(out.dtype, 0)
    need = query(M, N, K, sched, ab_t, c_t)["workspace_bytes"]
    ws = workspace(need, a.device) if need > 0 else None
    _check(_lib.ts_gemm_clocked(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                                a.stride(0), a.stride(1), b.stride(0), b.stride(1), out.stride(0), out.stride(1),
                                ab_t, c_t, ctypes.byref(s), _stream_handle(a.device), rec.data_ptr(), rec.shape[0],
                                ws.data_ptr() if ws is not None else None, need))
    return rec


def clock_ghz(rec) -> dict:
    """Shader clock per workgroup from a ts_gemm_clocked record (s_memtime ticks over
    100 MHz s_memrealtime ticks): mean / min / max over workgroups, in GHz."""
    r = rec.cpu().to(torch.float64)
    ticks = r[:, 1] - r[:, 0]
    secs = (r[:, 3] - r[:, 2]) / 100e6
    ok = secs > 0
    ghz = ticks[ok] / secs[ok] / 1e9
    return {"mean": float(ghz.mean()), "min": float(ghz.min()), "max": float(ghz.max()),
            "programs": int(ok.sum())}


def _probe_tflops(launch, iters: int, reps: int, device) -> float:
    q = query(256, 256, 256)
    sink = torch.empty(q["cu_count"] * 512, dtype=torch.float32, device=device)
    flops = ctypes.c_double(0.0)
    stream = _stream_handle(sink.device)
    _check(launch(iters, sink, flops, stream))
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(launch(iters, sink, flops, stream))
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def mfma_loop_tflops(iters: int = 20000, reps: int = 3, device: int | str = "cuda") -> float:
    """Sustained MFMA rate (TFLOP/s) of the no-memory probe, best of ``reps`` timed launches."""
    return _probe_tflops(lambda n, sink, flops, stream: _lib.ts_mfma_loop_probe(
        n, sink.data_ptr(), sink.numel(), ctypes.byref(flops), stream), iters, reps, device)


def mfma_phase_tflops(pattern: int, iters: int = 10000, reps: int = 3, device: int | str = "cuda") -> float:
    """MFMA rate (TFLOP/s) of the barrier-phase probe (ts_mfma_phase_probe), best of ``reps``."""
    return _probe_tflops(lambda n, sink, flops, stream: _lib.ts_mfma_phase_probe(
        n, pattern, sink.data_ptr(), sink.numel(), ctypes.byref(flops), stream), iters, reps, device)


def gemm_raw(a_ptr: int, b_ptr: int, c_ptr: int, M: int, N: int, K: int,
             strides=(None, 1, None, 1, None, 1), ab_dtype: int = TS_F16, c_dtype: int = TS_F16,
             schedule: Schedule | None = None, stream: int = 0) -> int:
    """Direct call of ts_gemm with integer pointers; returns the status code."""
    sam, sak, sbk, sbn, scm, scn = strides
    sam = K if sam is None else sam
    sbk = N if sbk is None else sbk
    scm = N if scm is None else scm
    s = (schedule or Schedule())._c()
    return _lib.ts_gemm(a_ptr, b_ptr, c_ptr, M, N, K, sam, sak, sbk, sbn, scm, scn,
                        ab_dtype, c_dtype, ctypes.byref(s), stream)


def query(M: int, N: int, K: int, schedule: Schedule | None = None,
          ab_dtype: int = TS_F16, c_dtype: int = TS_F16) -> dict:
    info = LaunchInfo()
    s = (schedule or Schedule())._c()
    _check(_lib.ts_query(M, N, K, ab_dtype, c_dtype, ctypes.byref(s), ctypes.byref(info)))
    return info.as_dict()


def schedule_trace(M: int, N: int, K: int, schedule: Schedule | None = None,
                   ab_dtype: int = TS_F16, c_dtype: int = TS_F16, device: int | str = "cuda"):
    """GPU-computed work sequence of every workgroup, as an int32 [rows, 5] CPU tensor."""
    info = query(M, N, K, schedule, ab_dtype, c_dtype)
    grid = info["grid"]
    rows = grid * info["trace_items"]
    out = torch.empty((max(rows, 1), 5), dtype=torch.int32, device=device)
    s = (schedule or Schedule())._c()
    _check(_lib.ts_schedule_trace(M, N, K, ab_dtype, c_dtype, ctypes.byref(s), out.data_ptr(), rows,
                                  _stream_handle(out.device)))
    torch.cuda.synchronize(out.device)
    return out[:rows].cpu()


def schedule_trace_host(M: int, N: int, K: int, schedule: Schedule, cu_count: int = 0,
                        programs_per_cu: int = 0, ab_dtype: int = TS_F16, c_dtype: int = TS_F16):
    """The same work sequence computed by the library on the CPU (no GPU needed).

    In persistent modes with num_programs == 0, cu_count * programs_per_cu stands
    in for the device's grid.
    """
    import numpy as np

    sized = schedule
    if schedule.mode != "tiled" and schedule.num_programs == 0:
        sized = dataclasses.replace(schedule, num_programs=cu_count * programs_per_cu)
    info = query(M, N, K, sized, ab_dtype, c_dtype)
    rows = info["grid"] * info["trace_items"]
    out = np.full((max(rows, 1), 5), -7, dtype=np.int32)
    s = schedule._c()
    _check(_lib.ts_schedule_trace_host(M, N, K, ab_dtype, c_dtype, ctypes.byref(s), cu_count,
                                       programs_per_cu, out.ctypes.data, rows))
    return out[:rows]
