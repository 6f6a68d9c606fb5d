#!/usr/bin/env python3
"""Benchmark of the tiled GEMM on one MI355X.

Workload (default): C[16384,16384] = A[16384,4096] @ B[4096,16384], fp16 inputs
drawn uniformly from [-1, 1) with a fixed seed, fp32 accumulation, fp16 output.
A step is one GEMM launch over device-resident inputs.  Prints one JSON line:
throughput (TFLOP/s = 2MNK / t), the roofline of the kernel (achieved vs MI355X
dense fp16 MFMA peak, from HIP events on the launch stream), the HBM traffic the
last hardware-counter profile measured for this kernel source, and the CPU
oracle's throughput on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--schedule S] [--workload NAME]
                    [--sweep] [--ksweep] [--extras] [--pps-sweep] [--index-ablation] [--pingpong-ab]
                    [--pmc-target | --stall-target | --target mix|ksweep|ragged]

--sweep times every order x remap x mode at the workload; --ksweep times the
grouped persistent loop against the flattened cross-tile loop over the K sweep
at 16384 x 16384; --extras times the benchmarked launch hot and cold, the 8192
grid, the ragged bf16 workload and one GPU's share of an eight-way row split,
and the oracle on one host thread (tables on stderr, before the JSON line).
--pps-sweep times one and two workgroups per CU for the 128x128x64 tile;
--index-ablation times the tile-order maps by division against multiply-shift;
--pingpong-ab times the ping-pong kernel against the 8-wave kernel and runs the
barrier-phase probe.
--pmc-target, --stall-target and --target only run the fixed launch sequences
that the hardware-counter passes profile.

Schedules are written order[+remap]/mode[/P<programs>][/tile], e.g.
"grouped8+remap/tiled", "rowmajor/persistent/P256", "grouped8/crosstile".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0     # MI355X dense fp16/bf16 MFMA
MFMA_TFLOPS_PER_GHZ = 256 * 4 * 1024 / 1000.0   # 256 CUs x 4 SIMDs x 1024 FLOP/clk, per GHz
PEAK_HBM_GBS = 8000.0    # MI355X HBM3E
METRIC = "fp16 GEMM TFLOPS (2MNK/s) + % MFMA peak at M=N=16384, K=4096"
DEFAULT_SCHEDULE = "auto/auto"   # order, G, remap and mode chosen by the library per shape
KERNEL_SOURCES = ["tile_scheduling_amd/csrc/gemm_kernel.hpp", "tile_scheduling_amd/csrc/schedule.hpp",
                  "tile_scheduling_amd/csrc/internal.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_schedule(text: str):
    import tile_scheduling_amd as ts

    parts = text.split("/")
    order_s = parts[0]
    remap = order_s.endswith("+remap")
    order_s = order_s.replace("+remap", "")
    if order_s in ("rowmajor", "row_major"):
        order, G = "row_major", 8
    elif order_s in ("auto", "autoorder"):
        order, G = "auto", 8
    else:
        m = re.fullmatch(r"grouped(\d+)", order_s)
        if not m:
            raise ValueError(f"bad order {order_s!r}")
        order, G = "grouped", int(m.group(1))
    mode = parts[1] if len(parts) > 1 else "tiled"
    P, tile, index_math = 0, "auto", "divide"
    for extra in parts[2:]:
        if extra.startswith("P"):
            P = int(extra[1:])
        elif extra in ("mulshift", "divide"):
            index_math = extra
        else:
            tile = extra
    return ts.Schedule(order=order, group_m=G, mode=mode, num_programs=P, xcd_remap=remap, tile=tile,
                       index_math=index_math)


def resolved_label(q) -> str:
    """The schedule ts_query resolved (auto order and mode replaced by the choice)."""
    o = f"grouped{q['group_m']}" if q["order"] == 1 else "rowmajor"
    r = "+remap" if q["xcd_remap"] else ""
    m = {0: "tiled", 1: "persistent", 2: "crosstile", 3: "streamk"}[q["mode"]]
    return f"{o}{r}/{m}"


def kernel_path(q, layout: str) -> int:
    """Kernel path of the launch: ts_query plans dense [M][K] / [K][N] operands; by the
    library's layout rules, whole tiles run path 3 with B stored [N][K], 4 with A
    stored [K][M] and 5 with both (on tiles with the direct-to-LDS pipeline), and
    anything else with a transposed operand the masked register path (1)."""
    if layout == "NN":
        return q["masked"]
    fast = q["masked"] == 0 and q["block_k"] == 64   # whole tiles on a direct-to-LDS configuration
    square = q["block_m"] == q["block_n"]
    if layout == "NT":
        return 3 if fast else 1
    if layout == "TN":
        return 4 if fast and square else 1
    return 5 if fast and square else 1


def sources_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sched_label: str):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_0-9]+):\s*(\S+)\s*$", line)
        if m:
            vals[m.group(1)] = m.group(2)
    if vals.get("source_sha") != sources_sha() or vals.get("schedule") != sched_label:
        return None
    try:
        return int(float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def time_gemm(ts, torch, a, b, c, sched, steps, warmup):
    for _ in range(warmup):
        ts.gemm(a, b, out=c, schedule=sched)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        ts.gemm(a, b, out=c, schedule=sched)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"wall_s": wall, "event_ms": ev[0].elapsed_time(ev[-1]) / steps, "median_ms": per[len(per) // 2],
            "min_ms": per[0], "p90_ms": per[min(steps - 1, (9 * steps) // 10)], "max_ms": per[-1]}


def time_gemm_cold(ts, torch, a, b, c, sched, steps, flush):
    """Per-launch event times with a 1 GiB write between launches (evicts the L2s and
    the Infinity Cache); the events bracket the GEMM alone."""
    stream = torch.cuda.current_stream()
    ts.gemm(a, b, out=c, schedule=sched)
    per = []
    for i in range(steps):
        flush.fill_(float(i & 7))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ts.gemm(a, b, out=c, schedule=sched)
        e1.record(stream)
        per.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in per)
    return {"median_ms": t[len(t) // 2], "min_ms": t[0], "p90_ms": t[min(steps - 1, (9 * steps) // 10)],
            "max_ms": t[-1]}


def cpu_baseline(A, B, w, budget_s: float, threads: int = 0):
    """The oracle on whole rows of C, sized to about budget_s seconds of host work."""
    from oracle import gemm as og

    threads = threads or max(1, min(16, os.cpu_count() or 1))
    rows = threads
    t0 = time.perf_counter()
    og.gemm(A, B, w.ab_dtype, rows=(0, rows), threads=threads)
    t_cal = time.perf_counter() - t0
    rows = int(min(w.M, max(threads, threads * round(budget_s / max(t_cal, 1e-6)))))
    t0 = time.perf_counter()
    og.gemm(A, B, w.ab_dtype, rows=(0, rows), threads=threads)
    t = time.perf_counter() - t0
    return {"value": round(2.0 * rows * w.N * w.K / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} full rows of C ({rows}x{w.N} outputs, K={w.K}, fp64 accumulation) "
                      f"in {t:.1f} s on {threads} threads"}


PMC_SCHEDULES = {
    "gemm_16384x16384x4096_f16": [f"{o}{r}/{m}" for o in ("rowmajor", "grouped4", "grouped8", "grouped16")
                                  for r in ("", "+remap") for m in ("tiled", "persistent")]
                                 + ["rowmajor/crosstile", "grouped8+remap/crosstile"],
    "gemm_8192x8192x4096_f16": [f"{o}{r}/{m}" for o in ("rowmajor", "grouped8")
                                for r in ("", "+remap") for m in ("tiled", "persistent")],
}


def pmc_target(ts, torch, np, workloads):
    """Launch sequence for counter passes: a fill and a copy of 1 GiB each (known
    HBM bytes, to scale the counters), then two launches of every schedule in
    PMC_SCHEDULES.  Prints a manifest line per dispatch in launch order."""
    n = 1 << 29  # 2-byte elements: 1 GiB per buffer
    x = torch.empty(n, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    torch.cuda.synchronize()
    print("dispatch fill 1073741824 write", flush=True)
    y.copy_(x)
    torch.cuda.synchronize()
    print("dispatch copy 1073741824 read+write", flush=True)
    del x, y
    by_name = {w.name: w for w in workloads.ALL}
    for name, labels in PMC_SCHEDULES.items():
        w = by_name[name]
        A, B = workloads.inputs(w)
        in_dtype = torch.float16 if w.ab_dtype == "f16" else torch.bfloat16
        a = torch.from_numpy(A.view(np.int16)).view(in_dtype).cuda()
        b = torch.from_numpy(B.view(np.int16)).view(in_dtype).cuda()
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        for lab in labels:
            s = parse_schedule(lab)
            for rep in range(2):
                ts.gemm(a, b, out=c, schedule=s)
                torch.cuda.synchronize()
                print(f"dispatch gemm {name} {s.label()} rep{rep}", flush=True)
        del a, b, c


STALL_SCHEDULES = ("grouped8+remap/persistent/256x256x64w8", "grouped8+remap/persistent/256x256x64",
                   "grouped8+remap/crosstile/256x256x64w8", "grouped8+remap/persistent/256x256x64pp")


def stall_target(ts, torch, np, workloads):
    """Launch sequence for the wave-state counter passes: three launches each of the
    8-wave and 4-wave 256x256x64 persistent kernels, the 8-wave cross-tile kernel and
    the ping-pong kernel at 16384 x 16384 x 4096.  Prints a manifest line per dispatch."""
    w = workloads.SQ_16384
    A, B = workloads.inputs(w)
    a = torch.from_numpy(A.view(np.int16)).view(torch.float16).cuda()
    b = torch.from_numpy(B.view(np.int16)).view(torch.float16).cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    for lab in STALL_SCHEDULES:
        s = parse_schedule(lab)
        for rep in range(3):
            ts.gemm(a, b, out=c, schedule=s)
            torch.cuda.synchronize()
            print(f"dispatch gemm {w.name} {s.label()} rep{rep}", flush=True)


def _device_inputs(ts, torch, np, w):
    A, B = __import__("workloads").inputs(w)
    in_dtype = torch.float16 if w.ab_dtype == "f16" else torch.bfloat16
    out_dtype = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.c_dtype]
    a = torch.from_numpy(A.view(np.int16)).view(in_dtype).cuda()
    b = torch.from_numpy(B.view(np.int16)).view(in_dtype).cuda()
    c = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda")
    return a, b, c


# Launch sequences for the other counter passes (`--target NAME`): each runs the
# listed (workload, schedule) launches `reps` times, synchronising after each, and
# prints one manifest line per dispatch, so that the profile's dispatch rows can
# be matched to schedules.
TARGETS = {
    # instruction mix: one tile per workgroup against the persistent loop, with the
    # tile-order maps by integer division and by multiply-shift
    "mix": [(w, f"grouped8+remap/{m}{x}") for w in ("gemm_4096x4096x4096_f16", "gemm_16384x16384x4096_f16")
            for m in ("tiled", "persistent") for x in ("", "/mulshift")],
    # the K sweep: grouped persistent against the flattened cross-tile loop
    "ksweep": [(f"gemm_16384x16384x{k}_f16_ksweep", f"grouped8+remap/{m}") for k in (128, 512, 1024, 2048, 4096)
               for m in ("persistent", "crosstile")],
    # the ragged bf16 product: persistent, cross-tile and stream-K on the edge path
    "ragged": [("gemm_5000x12290x1000_bf16_f32", f"grouped8+remap/{m}") for m in ("persistent", "crosstile",
                                                                                  "streamk")],
}


def scaling_dispatches(torch):
    """A 1 GiB fill and a 1 GiB copy (known HBM bytes, to scale FETCH_SIZE and
    WRITE_SIZE), each announced by a manifest line."""
    n = 1 << 29  # 2-byte elements: 1 GiB per buffer
    x = torch.empty(n, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    torch.cuda.synchronize()
    print("dispatch fill 1073741824 write", flush=True)
    y.copy_(x)
    torch.cuda.synchronize()
    print("dispatch copy 1073741824 read+write", flush=True)
    del x, y
    torch.cuda.empty_cache()


def run_target(ts, torch, np, workloads, name, reps=3):
    by_name = {w.name: w for w in workloads.ALL}
    scaling_dispatches(torch)
    loaded = {}
    for wname, lab in TARGETS[name]:
        if wname not in loaded:
            loaded.clear()
            torch.cuda.empty_cache()
            loaded[wname] = _device_inputs(ts, torch, np, by_name[wname])
        a, b, c = loaded[wname]
        s = parse_schedule(lab)
        for rep in range(reps):
            ts.gemm(a, b, out=c, schedule=s)
            torch.cuda.synchronize()
            print(f"dispatch gemm {wname} {s.label()} rep{rep}", flush=True)


def pps_sweep(ts, torch, np, workloads, steps):
    """Programs per CU (the persistent page's programs_per_sm): the 128 x 128 x 64
    tile (two workgroups fit a CU) with P = CUs x 1 and CUs x 2, against its tiled
    launch, at 4096^3 and 16384^2 x 4096 (stderr table)."""
    cus = ts.query(256, 256, 256)["cu_count"]
    for wname in ("gemm_4096x4096x4096_f16", "gemm_16384x16384x4096_f16"):
        w = {x.name: x for x in workloads.ALL}[wname]
        a, b, c = _device_inputs(ts, torch, np, w)
        flops = 2.0 * w.M * w.N * w.K
        for lab in ["grouped8+remap/tiled/128x128x64"] + \
                   [f"grouped8+remap/persistent/P{cus * k}/128x128x64" for k in (1, 2)] + \
                   ["grouped8+remap/persistent/256x256x64w8"]:
            s = parse_schedule(lab)
            r = time_gemm(ts, torch, a, b, c, s, steps, 10)
            q = ts.query(w.M, w.N, w.K, s)
            log(f"pps {wname} {lab:44s} grid {q['grid']:5d} ({q['programs_per_cu']} per CU fit)  "
                f"median {r['median_ms']:.4f} ms  {flops / r['median_ms'] / 1e9:8.1f} TFLOP/s")
        del a, b, c


def index_ablation(ts, torch, np, workloads, steps):
    """Tile-order maps by integer division against multiply-shift (stderr table)."""
    for wname in ("gemm_4096x4096x4096_f16", "gemm_16384x16384x4096_f16", "gemm_16384x16384x128_f16_ksweep"):
        w = {x.name: x for x in workloads.ALL}[wname]
        a, b, c = _device_inputs(ts, torch, np, w)
        flops = 2.0 * w.M * w.N * w.K
        for m in ("tiled", "persistent", "crosstile"):
            for x in ("", "/mulshift"):
                lab = f"grouped8+remap/{m}{x}"
                r = time_gemm(ts, torch, a, b, c, parse_schedule(lab), steps, 10)
                log(f"index {wname} {lab:36s} median {r['median_ms']:.4f} ms (p90 {r['p90_ms']:.4f})  "
                    f"{flops / r['median_ms'] / 1e9:8.1f} TFLOP/s")
        del a, b, c


def pingpong_ab(ts, torch, np, workloads, steps):
    """The ping-pong kernel against the 8-wave kernel of the same tile, launches
    interleaved per workload, and the barrier-phase probe (stderr table)."""
    for pat, what in ((0, "no barrier"), (1, "barrier every 8 MFMAs, all waves"),
                      (2, "ping-pong, 16-MFMA phases"), (3, "ping-pong, 32-MFMA phases")):
        log(f"phase-probe pattern {pat} ({what}): {ts.mfma_phase_tflops(pat):8.1f} TFLOP/s")
    names = ["gemm_16384x16384x4096_f16", "gemm_8192x8192x4096_f16", "gemm_16384x16384x4096_bf16",
             "gemm_16384x16384x128_f16_ksweep", "gemm_16384x16384x1024_f16_ksweep", "gemm_5000x12290x1000_bf16_f32"]
    by = {x.name: x for x in workloads.ALL}
    for wname in names:
        w = by[wname]
        a, b, c = _device_inputs(ts, torch, np, w)
        flops = 2.0 * w.M * w.N * w.K
        for mode in ("persistent", "crosstile"):
            labs = [f"grouped8+remap/{mode}/256x256x64w8", f"grouped8+remap/{mode}/256x256x64pp"]
            res = {lab: [] for lab in labs}
            for _ in range(3):   # interleaved, so that both see the same clock drift
                for lab in labs:
                    res[lab].append(time_gemm(ts, torch, a, b, c, parse_schedule(lab), steps, 10)["median_ms"])
            for lab in labs:
                ms = sorted(res[lab])[1]
                log(f"pingpong {wname} {lab:40s} median of 3 medians {ms:.4f} ms  "
                    f"{flops / ms / 1e9:8.1f} TFLOP/s")
        del a, b, c


KSWEEP_SCHEDULES = ("grouped8+remap/persistent", "grouped8+remap/crosstile")


def ksweep(ts, torch, np, workloads, steps):
    """Grouped persistent vs persistent + cross-tile over the K sweep (stderr table)."""
    for w in workloads.K_SWEEP:
        A, B = workloads.inputs(w)
        a = torch.from_numpy(A.view(np.int16)).view(torch.float16).cuda()
        b = torch.from_numpy(B.view(np.int16)).view(torch.float16).cuda()
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        flops = 2.0 * w.M * w.N * w.K
        hbm = 2.0 * (w.M * w.K + w.K * w.N + w.M * w.N)   # compulsory bytes, fp16
        for lab in KSWEEP_SCHEDULES:
            r = time_gemm(ts, torch, a, b, c, parse_schedule(lab), steps, 10)
            t = r["median_ms"] * 1e-3
            log(f"ksweep K={w.K:5d} {lab:28s} median {r['median_ms']:.4f} ms (min {r['min_ms']:.4f}, "
                f"p90 {r['p90_ms']:.4f})  {flops / t / 1e12:8.1f} TFLOP/s  compulsory {hbm / t / 1e9:7.1f} GB/s")
        del a, b, c


EXTRA_SETS = (
    # (workload, schedules): the 8192 grid, every order x mode on the ragged bf16 shape,
    # one GPU's share of an eight-way row split of the headline product, 4096 cubed, and
    # the headline shape in bf16 and with fp32 output
    ("gemm_8192x8192x4096_f16", [f"{o}{r}/{m}" for o in ("rowmajor", "grouped8") for r in ("", "+remap")
                                 for m in ("tiled", "persistent", "crosstile")]),
    ("gemm_5000x12290x1000_bf16_f32", [f"{o}{r}/{m}" for o in ("rowmajor", "grouped4", "grouped8", "grouped16")
                                       for r in ("", "+remap") for m in ("tiled", "persistent", "crosstile")]),
    ("gemm_2048x16384x4096_f16_mshare8", [f"{o}/{m}" for o in ("rowmajor", "grouped8+remap")
                                          for m in ("tiled", "persistent", "crosstile")]),
    ("gemm_4096x4096x4096_f16", [f"{o}/{m}" for o in ("rowmajor", "grouped8+remap") for m in ("tiled", "persistent")]
     + ["grouped8+remap/crosstile", "grouped8+remap/tiled/128x128x64", "grouped8+remap/persistent/128x128x64"]),
    ("gemm_16384x16384x4096_bf16", ["grouped8+remap/persistent", "grouped8+remap/crosstile"]),
    ("gemm_16384x16384x4096_f16_f32", ["grouped8+remap/persistent", "grouped8+remap/crosstile"]),
)


def extras(ts, torch, np, workloads, a, b, c, w, sched, steps):
    """Supplementary tables on stderr: hot and cold-cache timing of the benchmarked
    launch, the other workloads' schedules (useful and executed TFLOP/s), and the
    oracle on one host thread."""
    flops = 2.0 * w.M * w.N * w.K
    flush = torch.empty(1 << 29, dtype=torch.float16, device="cuda")
    hot = time_gemm(ts, torch, a, b, c, sched, steps, 3)
    cold = time_gemm_cold(ts, torch, a, b, c, sched, steps, flush)
    for name, r in (("hot", hot), ("cold", cold)):
        log(f"extras {w.name} {sched.label()} {name:4s} median {r['median_ms']:.4f} ms "
            f"(min {r['min_ms']:.4f}, p90 {r['p90_ms']:.4f}, max {r['max_ms']:.4f})  "
            f"{flops / r['median_ms'] / 1e9:8.1f} TFLOP/s")
    del flush
    by_name = {x.name: x for x in workloads.ALL}
    for name, labels in EXTRA_SETS:
        x = by_name[name]
        A, B = workloads.inputs(x)
        in_dtype = torch.float16 if x.ab_dtype == "f16" else torch.bfloat16
        out_dtype = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[x.c_dtype]
        xa = torch.from_numpy(A.view(np.int16)).view(in_dtype).cuda()
        xb = torch.from_numpy(B.view(np.int16)).view(in_dtype).cuda()
        xc = torch.empty((x.M, x.N), dtype=out_dtype, device="cuda")
        useful = 2.0 * x.M * x.N * x.K
        for lab in labels:
            s = parse_schedule(lab)
            q = ts.query(x.M, x.N, x.K, s, ts.TS_F16 if x.ab_dtype == "f16" else ts.TS_BF16,
                         {"f16": ts.TS_F16, "bf16": ts.TS_BF16, "f32": ts.TS_F32}[x.c_dtype])
            executed = 2.0 * (q["num_m_tiles"] * q["block_m"]) * (q["num_n_tiles"] * q["block_n"]) * \
                (q["k_steps"] * q["block_k"])
            r = time_gemm(ts, torch, xa, xb, xc, s, steps, 3)
            t = r["median_ms"] * 1e-3
            log(f"extras {x.name} {lab:28s} tile {q['block_m']}x{q['block_n']}x{q['block_k']} grid {q['grid']:5d}  "
                f"median {r['median_ms']:.4f} ms (p90 {r['p90_ms']:.4f})  {useful / t / 1e12:7.1f} TFLOP/s useful  "
                f"{executed / t / 1e12:7.1f} executed")
        del xa, xb, xc
    A, B = workloads.inputs(w)
    one = cpu_baseline(A, B, w, 3.0, threads=1)
    log(f"extras oracle one thread: {one['value'] * 1e3:.3f} GFLOP/s ({one['sample']})")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the shader clock settles over the first few dozen launches (the board's power
    # management); the defaults time 100 launches after 50 untimed ones
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gemm_16384x16384x4096_f16")
    ap.add_argument("--layout", default="NN", choices=["NN", "NT", "TN", "TT"],
                    help="operand storage: A [M][K] (N) or [K][M] (T), B [K][N] (N) or [N][K] (T)")
    ap.add_argument("--schedule", default=DEFAULT_SCHEDULE)
    ap.add_argument("--sweep", action="store_true", help="also time every schedule (table on stderr)")
    ap.add_argument("--ksweep", action="store_true",
                    help="also time persistent vs cross-tile over the K sweep (table on stderr)")
    ap.add_argument("--extras", action="store_true",
                    help="also print hot/cold timing, the other workloads' schedules and the "
                         "one-thread oracle rate (tables on stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-target", action="store_true",
                    help="run the fixed launch sequence used for hardware-counter passes and exit")
    ap.add_argument("--stall-target", action="store_true",
                    help="run the launch sequence of the wave-state counter passes and exit")
    ap.add_argument("--target", choices=sorted(TARGETS),
                    help="run one of the other counter-pass launch sequences and exit")
    ap.add_argument("--pps-sweep", action="store_true",
                    help="also time programs per CU 1 and 2 for the 128x128x64 tile (stderr table)")
    ap.add_argument("--index-ablation", action="store_true",
                    help="also time the tile maps by integer division against multiply-shift (stderr table)")
    ap.add_argument("--pingpong-ab", action="store_true",
                    help="also time the ping-pong kernel against the 8-wave kernel and run the "
                         "barrier-phase probe (stderr table)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the GEMM runs on one GPU; a multi-GPU split by rows of A and C is not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tile_scheduling_amd as ts
    import workloads

    by_name = {w.name: w for w in workloads.ALL}
    if args.pmc_target:
        pmc_target(ts, torch, np, workloads)
        return
    if args.stall_target:
        stall_target(ts, torch, np, workloads)
        return
    if args.target:
        run_target(ts, torch, np, workloads, args.target)
        return
    w = by_name[args.workload]
    out_dtype = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.c_dtype]
    in_dtype = torch.float16 if w.ab_dtype == "f16" else torch.bfloat16

    A, B = workloads.inputs(w)
    if args.layout[0] == "T":   # A stored [K][M]: the same values through a transposed view
        a = torch.from_numpy(np.ascontiguousarray(A.T).view(np.int16)).view(in_dtype).cuda().t()
    else:
        a = torch.from_numpy(A.view(np.int16)).view(in_dtype).cuda()
    if args.layout[1] == "T":   # B stored [N][K]
        b = torch.from_numpy(np.ascontiguousarray(B.T).view(np.int16)).view(in_dtype).cuda().t()
    else:
        b = torch.from_numpy(B.view(np.int16)).view(in_dtype).cuda()
    c = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda")
    flops = 2.0 * w.M * w.N * w.K

    if args.ksweep:
        ksweep(ts, torch, np, workloads, max(10, args.steps))
    if args.pps_sweep:
        pps_sweep(ts, torch, np, workloads, max(10, args.steps))
    if args.index_ablation:
        index_ablation(ts, torch, np, workloads, max(10, args.steps))
    if args.pingpong_ab:
        pingpong_ab(ts, torch, np, workloads, max(10, args.steps))
    if args.extras:
        extras(ts, torch, np, workloads, a, b, c, w, parse_schedule(args.schedule), max(10, args.steps))
    if args.sweep:
        labels = []
        for order in ("rowmajor", "grouped4", "grouped8", "grouped16"):
            for remap in ("", "+remap"):
                for mode in ("tiled", "persistent", "crosstile"):
                    labels.append(f"{order}{remap}/{mode}")
        for lab in labels:
            s = parse_schedule(lab)
            r = time_gemm(ts, torch, a, b, c, s, max(5, args.steps // 2), 2)
            log(f"sweep {w.name} {lab:28s} median {r['median_ms']:.4f} ms  "
                f"{flops / r['median_ms'] / 1e9:9.1f} TFLOP/s")

    sched = parse_schedule(args.schedule)
    q = ts.query(w.M, w.N, w.K, sched, ts.TS_F16 if w.ab_dtype == "f16" else ts.TS_BF16,
                 {"f16": ts.TS_F16, "bf16": ts.TS_BF16, "f32": ts.TS_F32}[w.c_dtype])
    log(f"launch {sched.label()}: {q}")
    r = time_gemm(ts, torch, a, b, c, sched, args.steps, args.warmup)
    ms_per_step = r["wall_s"] * 1e3 / args.steps
    value = flops * args.steps / r["wall_s"] / 1e12
    achieved = flops / (r["event_ms"] * 1e-3) / 1e12
    log(f"timed {args.steps} steps: wall {ms_per_step:.4f} ms/step, events {r['event_ms']:.4f} ms/launch "
        f"(median {r['median_ms']:.4f}, min {r['min_ms']:.4f}, p90 {r['p90_ms']:.4f}, max {r['max_ms']:.4f})")

    # One more launch with the per-workgroup clock record, outside the timed region:
    # the shader clock the board's power limit allowed, and the MFMA peak at it.
    clk = ts.clock_ghz(ts.gemm_clocked(a, b, c, schedule=sched))
    torch.cuda.synchronize()
    peak_at_clock = MFMA_TFLOPS_PER_GHZ * clk["mean"]
    clock = {"ghz": round(clk["mean"], 4), "ghz_min": round(clk["min"], 4), "ghz_max": round(clk["max"], 4),
             "mfma_peak_at_clock": round(peak_at_clock, 1), "frac_at_clock": round(achieved / peak_at_clock, 4),
             "source": "s_memtime over s_memrealtime (100 MHz) per workgroup, one launch after the timed ones; "
                       "loop peak: no-memory MFMA probe, 8 waves per CU"}
    loop_peak = ts.mfma_loop_tflops()
    clock["mfma_loop_peak"] = round(loop_peak, 1)
    clock["frac_of_loop_peak"] = round(achieved / loop_peak, 4)
    log(f"clock {clock}")

    traffic = measured_traffic(w.name, resolved_label(q))
    # Roofline of the workload: compulsory bytes (A and B read once, C written once)
    # against 2MNK; below the ridge point (peak FLOP/s over peak bytes/s) the kernel
    # is bound by HBM and is reported against the HBM roof.
    esz = {"f16": 2, "bf16": 2, "f32": 4}
    compulsory = esz[w.ab_dtype] * (w.M * w.K + w.K * w.N) + esz[w.c_dtype] * w.M * w.N
    intensity = flops / compulsory
    ridge = PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        gbs = compulsory / (r["event_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1)}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1)}
    executed = 2.0 * (q["num_m_tiles"] * q["block_m"]) * (q["num_n_tiles"] * q["block_n"]) * \
        (max(q["k_steps"], 1) * q["block_k"])
    metric = METRIC if w.name == workloads.SQ_16384.name else \
        f"{w.ab_dtype} GEMM TFLOPS (2MNK/s) + % of roofline at M={w.M}, N={w.N}, K={w.K}"

    result = {
        "metric": metric, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.ab_dtype, "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": args.layout, "in": w.ab_dtype,
                   "acc": "f32",
                   "out": w.c_dtype, "inputs": f"{w.dist} seed {w.seed}", "schedule": sched.label(),
                   "resolved_schedule": resolved_label(q),
                   "tile": f"{q['block_m']}x{q['block_n']}x{q['block_k']}", "threads": q["threads"],
                   "grid": q["grid"], "kernel_path": kernel_path(q, args.layout),
                   "executed_tflops": round(executed * args.steps / r["wall_s"] / 1e12, 2)},
        "roofline": roof,
        "clock": clock,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(A, B, w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
