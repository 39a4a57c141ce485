#!/usr/bin/env python3
"""Benchmark of the FP16 linear layer y = FP16(FP16(x @ weight.T) + b) on one MI355X.

One step is the decode-shaped GEMV batch: the layer at x [1, 4096] and at
x [16, 4096], each against a [4096, 4096] weight and a [4096] bias (both calls
go through the library's automatic path choice, i.e. the skinny
weight-streaming kernel).  The metric is HBM GB/s from algorithmic bytes
(x, weight and b read once, y written once).  Weight copies rotate over more
than 512 MiB so the 256 MB Infinity Cache cannot serve a weight from a previous
call.  Inputs are synthetic, seeded, resident in HBM before timing starts.

The line also carries, under "prefill", the MFMA-bound shapes (toy 1024x1024x768,
attention projection 8192x4096x4096, MLP up-projection 4096x14336x4096, ragged
down-projection 2000x4000x14336) in TFLOP/s against the FP16 dense MFMA peak;
under "variants", the bfloat16, FP32-output and epilogue-program forms, the
grouped contraction (8 x 512x4096x4096) and the indexed contraction
(moe_decode: 32 rows over 8 experts of [4096, 4096]; moe_prefill: 4096 rows);
under "cpu_baseline", the CPU oracle timed on this host; and, under "context",
the per-launch floor of the smallest call and one decode call timed alone.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-variants] [--no-cpu]
       python bench.py --only <workload> [--variant V]   (one workload alone, for profiling)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPYCAL_BYTES = (64 << 20) * 4   # one copy in --only copycal: 64 Mi float32 read and written
# sources whose change invalidates recorded counter readings, per kernel
KERNEL_SOURCES = {
    "decode_f16_step": ["linear_amd/csrc/skinny.hip", "linear_amd/csrc/common.h"],
    "gemm_f16_stream": ["linear_amd/csrc/gemm_impl.h", "linear_amd/csrc/gemm_f16.hip",
                        "linear_amd/csrc/common.h"],
}
# substrings of the demangled kernel names whose counter rows a record averages
# over (per dispatch)
KERNEL_PATTERNS = {
    # the decode step's two launches, binary16 with the bias step: M = 1 on the
    # one-row kernel, M = 16 on the 16-row kernel (8 waves)
    "decode_f16_step": ("gemv_stream<0, 0>", "skinny_stream<8, 0, 0>"),
    "gemm_f16_stream": ("gemm_stream<",),
}
MFMA_F16_PEAK_TFLOPS = 2516.6   # MI355X dense FP16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
ROTATE_BYTES = 512 * 1024 * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--repeats", type=int, default=1, help="timed regions of --steps steps each; the median is reported")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="time only this workload (profiling runs)")
    ap.add_argument("--variant", default="f16", help="with --only: f16, bf16, f16_f32out, bf16_f32out or "
                    "<f16|bf16>_epi_<gelu|res|silu_mul|silu>; f16 or bf16 for grouped, moe_decode, moe_prefill")
    ap.add_argument("--no-variants", action="store_true", help="skip the bfloat16 / FP32-output timings")
    ap.add_argument("--record-traffic", nargs=5, metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR"),
                    help="store HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE CSV runs")
    return ap.parse_args()


def sources_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_means(csv_dir: str, counter: str):
    """Mean per-dispatch value of `counter` for each kernel in a rocprofv3 --pmc CSV."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in out.items()}


def record_traffic(kernel: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                   commands: list[str]):
    """Turn FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of `kernel` and of the plain
    copy calibration into bytes per launch, and store them with a hash of the kernel
    sources so that a later change of the kernel invalidates them.  A record over
    several kernels (KERNEL_PATTERNS) averages their per-dispatch means."""
    def pick(d, counter, names):
        if isinstance(names, str):
            names = (names,)
        m = _counter_means(d, counter)
        hits = [(k, v) for k, v in m.items() if any(n in k for n in names)]
        if not hits:
            raise SystemExit("no %s dispatches of %s under %s" % (counter, " or ".join(names), d))
        # each matching kernel counts once (one launch each per unit of work, e.g.
        # the decode step's M = 1 and M = 16 calls), whatever its dispatch count
        n = sum(c for _, (_, c) in hits)
        mean = sum(v for _, (v, _) in hits) / len(hits)
        return " + ".join(sorted(k for k, _ in hits)), (mean, n)
    kname, (fetch_kib, nf) = pick(fetch_dir, "FETCH_SIZE", KERNEL_PATTERNS[kernel])
    _, (write_kib, nw) = pick(write_dir, "WRITE_SIZE", KERNEL_PATTERNS[kernel])
    _, (cf_kib, _) = pick(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    _, (cw_kib, _) = pick(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f_scale = COPYCAL_BYTES / (cf_kib * 1024.0)
    w_scale = COPYCAL_BYTES / (cw_kib * 1024.0)
    rec = {}
    if os.path.exists(TRAFFIC_JSON):
        rec = json.load(open(TRAFFIC_JSON))
    rec[kernel] = {
        "kernel_name": kname,
        "fetch_kib_per_dispatch": round(fetch_kib, 1),
        "write_kib_per_dispatch": round(write_kib, 1),
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": COPYCAL_BYTES, "fetch_kib": round(cf_kib, 1), "write_kib": round(cw_kib, 1),
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "bytes_per_launch": round(fetch_kib * 1024.0 * f_scale + write_kib * 1024.0 * w_scale),
        "sources_sha": sources_hash(kernel),
        "commands": commands,
    }
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec[kernel]))


def recorded_traffic(kernel: str):
    """Bytes per launch from the counter runs, or None if absent or the kernel changed since."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha") != sources_hash(kernel):
        return None
    return rec["bytes_per_launch"]


def rotation_sets(bytes_per_set: int) -> int:
    return max(2, math.ceil(ROTATE_BYTES / max(bytes_per_set, 1)))


def graph_calls(sets: int, minimum: int = 64) -> int:
    """Calls per captured graph: a multiple of the input sets (each used equally)
    and at least `minimum`, since every replay adds a graph launch of its own."""
    return sets * max(1, math.ceil(minimum / sets))


def capture(fn, calls, stream, torch):
    """Capture fn(0) .. fn(calls-1) into one HIP graph on `stream` (launch overhead of
    Python and ctypes stays out of the timed region; the kernels allocate nothing
    and issue no memset, so they replay unchanged)."""
    with torch.cuda.stream(stream):
        for i in range(calls):      # eager warm-up on the capture stream
            fn(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(calls):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_region(graph, replays, stream, torch):
    """Replay `graph` `replays` times between two HIP events on `stream`; return ms."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(replays):
            graph.replay()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end)


STEPS_PER_GRAPH = 128   # decode steps per captured graph (each replay adds a graph launch of its own)


def step_schedule(steps: int, period: int):
    """How `steps` steps run as graph replays: (full replays of a `period`-step
    graph, steps in one remainder graph).  Always exactly `steps` steps."""
    steps = max(0, int(steps))
    return steps // period, steps % period


class StepRunner:
    """Runs exactly n decode steps as replays of one `period`-step graph plus one
    remainder graph (captured on first use).  Steps start at step 0 of the weight
    rotation in each graph; the period is a multiple of the rotation, so whole
    replays continue it seamlessly."""

    def __init__(self, step, period, stream, torch):
        self.step, self.period, self.stream, self.torch = step, period, stream, torch
        self.graphs = {}
        self.eager_steps = 0   # steps run eagerly while capturing (graph warm-up)

    def graph(self, n):
        if n not in self.graphs:
            self.graphs[n] = capture(self.step, n, self.stream, self.torch)
            self.eager_steps += n
        return self.graphs[n]

    def prepare(self, *counts):
        for c in counts:
            q, r = step_schedule(c, self.period)
            if q:
                self.graph(self.period)
            if r:
                self.graph(r)

    def run(self, n):
        q, r = step_schedule(n, self.period)
        for _ in range(q):
            self.graph(self.period).replay()
        if r:
            self.graph(r).replay()


def bench_decode(args, torch, la, workloads, stream, dtype=None):
    """The step: one call at M=1 and one at M=16.  Exactly args.warmup untimed
    steps, then timed regions of exactly args.steps steps each (args.repeats of
    them, the median reported; one by default).  Returns (ms_per_step, detail)."""
    dtype = dtype or torch.float16
    fn = la.linear_bf16 if dtype == torch.bfloat16 else la.linear_f16
    w1, w16 = workloads.WORKLOADS["gemv1"], workloads.WORKLOADS["gemv16"]
    x1, wbase, b = workloads.workload_inputs("gemv1", seed=0, device="cuda", dtype=dtype)
    x16, _, _ = workloads.workload_inputs("gemv16", seed=0, device="cuda", dtype=dtype)
    copies = rotation_sets(wbase.numel() * 2)
    weights = [wbase] + [wbase.clone() for _ in range(copies - 1)]
    y1 = torch.empty((1, w1.N), dtype=dtype, device="cuda")
    y16 = torch.empty((16, w16.N), dtype=dtype, device="cuda")
    step_bytes = w1.bytes + w16.bytes

    def step(i):
        fn(x1, weights[(2 * i) % copies], b, out=y1, stream=stream)
        fn(x16, weights[(2 * i + 1) % copies], b, out=y16, stream=stream)

    # a graph of a fixed number of steps, a multiple of copies / 2 so that whole
    # replays use every weight copy equally: the per-replay graph launch is then
    # the same fraction of a step whatever --steps asks for
    base = max(1, copies // 2)
    period = max(base, (STEPS_PER_GRAPH // base) * base)
    runner = StepRunner(step, period, stream, torch)
    runner.prepare(args.warmup, args.steps)
    torch.cuda.synchronize()
    runner.run(args.warmup)
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, args.repeats)):
        times.append(time_steps(runner, args.steps, stream, torch))
    ms = sorted(times)[len(times) // 2] / max(1, args.steps)
    q, r = step_schedule(args.steps, period)
    plan = la.linear_f16_plan(x16, wbase, b)
    detail = {
        "step_bytes": step_bytes,
        "weight_copies": copies,
        "steps_per_graph": period,
        "graph_replays": {"full": q, "remainder_steps": r},
        "timed_regions": len(times),
        "eager_steps_at_capture": runner.eager_steps,
        "ms_per_step_all": [t / max(1, args.steps) for t in times],
        "plan_m16": plan,
        "plan_m1": la.linear_f16_plan(x1, wbase, b),
    }
    del runner
    torch.cuda.synchronize()
    return ms, detail


def time_steps(runner, steps, stream, torch):
    """Exactly `steps` steps between two HIP events on `stream`, with the device
    synchronised on both sides; returns ms.  A region carries a fixed cost of
    about 10 us (its graphs' launch boundaries and the first steps after the idle
    device), 2.5-3% of a 20-step region and under 0.1% of a 2000-step one."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        runner.run(steps)
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def bench_context(torch, la, workloads, stream):
    """Context for the decode figures, not part of `value`: the per-launch floor of
    the smallest call (1 x 16 x 32, one workgroup) replayed in a graph, and one
    decode call (M = 1) timed alone between two events.  Every tensor a graph or a
    call uses stays referenced here until its last replay has finished."""
    log("context: launch floor (1 x 16 x 32 in a graph)")
    x = torch.ones((1, 32), dtype=torch.float16, device="cuda")
    w = torch.ones((16, 32), dtype=torch.float16, device="cuda")
    b = torch.zeros((16,), dtype=torch.float16, device="cuda")
    y = torch.empty((1, 16), dtype=torch.float16, device="cuda")
    g = capture(lambda i: la.linear_f16(x, w, b, out=y, stream=stream), 64, stream, torch)
    g.replay()
    floor = sorted(time_region(g, 20, stream, torch) / (20 * 64) for _ in range(5))[2] * 1e3
    torch.cuda.synchronize()
    del g

    log("context: single gemv1 calls")
    x1, w1, b1 = workloads.workload_inputs("gemv1", seed=0, device="cuda")
    y1 = torch.empty((1, w1.shape[0]), dtype=torch.float16, device="cuda")
    singles = []
    for _ in range(60):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            la.linear_f16(x1, w1, b1, out=y1, stream=stream)
            end.record(stream)
        end.synchronize()
        singles.append(start.elapsed_time(end) * 1e3)
    singles = sorted(singles[10:])
    return {"launch_floor_us": round(floor, 3),
            "single_call_gemv1_us": {"median": round(singles[len(singles) // 2], 3), "min": round(singles[0], 3)}}


# epilogue programs timed by the bench: name -> (steps, reads a residual, reads a gate input)
EPI_PROGRAMS = {
    "gelu": ("EPI_BIAS EPI_GELU_TANH", False, False),
    "res": ("EPI_BIAS EPI_RESIDUAL", True, False),
    "silu_mul": ("EPI_SILU EPI_MUL", False, True),
    "silu": ("EPI_BIAS EPI_SILU", False, False),
}


def bench_gemm(name, torch, la, workloads, stream, calls, variant="f16"):
    """One prefill shape.  variant: "f16" (the layer), "bf16" (bfloat16 layer),
    "f16_f32out" / "bf16_f32out" (the unrounded FP32 sums, no bias) or
    "<f16|bf16>_epi_<program>" (an epilogue program of EPI_PROGRAMS)."""
    wl = workloads.WORKLOADS[name]
    dtype = torch.bfloat16 if variant.startswith("bf16") else torch.float16
    sums = variant.endswith("f32out")
    prog = variant.split("_epi_", 1)[1] if "_epi_" in variant else None
    x, w, b = workloads.workload_inputs(name, seed=0, device="cuda", dtype=dtype)
    # algorithmic bytes: FP32 output is 4 B per element and there is no bias; an
    # epilogue reads its [M, N] inputs once (2 B per element each)
    nbytes = wl.bytes + (2 * wl.M * wl.N - 2 * wl.N if sums else 0)
    ops, r_in, u_in = [], False, False
    if prog:
        names, r_in, u_in = EPI_PROGRAMS[prog]
        ops = [getattr(la, n) for n in names.split()]
        nbytes += 2 * wl.M * wl.N * (int(r_in) + int(u_in)) - (0 if la.EPI_BIAS in ops else 2 * wl.N)
    sets = rotation_sets(nbytes)
    xs = [x] + [x.clone() for _ in range(sets - 1)]
    ws = [w] + [w.clone() for _ in range(sets - 1)]
    ys = [torch.empty((wl.M, wl.N), dtype=torch.float32 if sums else dtype, device="cuda")
          for _ in range(sets)]
    if sums:
        fn = la.linear_bf16_f32out if dtype == torch.bfloat16 else la.linear_f16_f32out
    elif prog:
        fn = la.linear_bf16_epilogue if dtype == torch.bfloat16 else la.linear_f16_epilogue
    else:
        fn = la.linear_bf16 if dtype == torch.bfloat16 else la.linear_f16
    g = torch.Generator(device="cpu").manual_seed(1)
    rs = [torch.randn(wl.M, wl.N, generator=g).to(dtype).to("cuda") for _ in range(sets)] if r_in else None
    us = [torch.rand(wl.M, wl.N, generator=g).to(dtype).to("cuda") for _ in range(sets)] if u_in else None
    if prog:   # builds the activation tables outside the capture
        fn(xs[0], ws[0], ops, bias=b, residual=rs[0] if rs else None, mul=us[0] if us else None, out=ys[0])
        torch.cuda.synchronize()

    def call(i):
        k = i % sets
        if sums:
            fn(xs[k], ws[k], out=ys[k], stream=stream)
        elif prog:
            fn(xs[k], ws[k], ops, bias=b, residual=rs[k] if rs else None, mul=us[k] if us else None, out=ys[k],
               stream=stream)
        else:
            fn(xs[k], ws[k], b, out=ys[k], stream=stream)

    per_graph = graph_calls(sets)
    graph = capture(call, per_graph, stream, torch)
    replays = max(1, calls // per_graph)
    graph.replay()
    times = [time_region(graph, replays, stream, torch) for _ in range(5)]
    ms = sorted(times)[len(times) // 2] / (replays * per_graph)
    del graph
    tflops = wl.flops / (ms * 1e-3) / 1e12
    plan = la.linear_f16_plan(x, w, b)
    del xs, ws, ys, rs, us
    return {
        "M": wl.M, "N": wl.N, "K": wl.K, "variant": variant,
        "us_per_call": round(ms * 1e3, 3),
        "tflops": round(tflops, 1),
        "frac_mfma_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "hbm_gbs_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "input_sets": sets,
        "tile": [plan["tile_m"], plan["tile_n"]],
        "grid": plan["grid"],
    }


def bench_grouped(name, torch, la, workloads, stream, calls, dtype_name="f16"):
    """The grouped contraction workload (G groups), in TFLOP/s."""
    wl = workloads.GROUPED[name]
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float16
    fn = la.linear_bf16_grouped if dtype == torch.bfloat16 else la.linear_f16_grouped
    x, w, b = workloads.make_grouped_inputs(wl.G, wl.M, wl.N, wl.K, wl.a, seed=0, device="cuda", dtype=dtype)
    sets = rotation_sets(wl.bytes)
    xs = [x] + [x.clone() for _ in range(sets - 1)]
    ws = [w] + [w.clone() for _ in range(sets - 1)]
    ys = [torch.empty((wl.G, wl.M, wl.N), dtype=dtype, device="cuda") for _ in range(sets)]

    def call(i):
        k = i % sets
        fn(xs[k], ws[k], b, out=ys[k], stream=stream)

    per_graph = graph_calls(sets)
    graph = capture(call, per_graph, stream, torch)
    replays = max(1, calls // per_graph)
    graph.replay()
    times = [time_region(graph, replays, stream, torch) for _ in range(5)]
    ms = sorted(times)[len(times) // 2] / (replays * per_graph)
    del graph, xs, ws, ys
    return {"G": wl.G, "M": wl.M, "N": wl.N, "K": wl.K, "variant": dtype_name,
            "us_per_call": round(ms * 1e3, 3), "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 1),
            "frac_mfma_peak": round(wl.flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4), "input_sets": sets}


def bench_indexed(name, torch, la, workloads, stream, calls, dtype_name="f16"):
    """The indexed (expert) contraction: TFLOP/s, and HBM GB/s over the algorithmic
    bytes (x, the tables of the experts idx selects, idx, y)."""
    wl = workloads.INDEXED[name]
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float16
    fn = la.linear_bf16_indexed if dtype == torch.bfloat16 else la.linear_f16_indexed
    x, w, idx = workloads.make_indexed_inputs(wl.E, wl.M, wl.N, wl.K, wl.a, seed=0, device="cuda", dtype=dtype)
    used = int(torch.unique(idx).numel())
    nbytes = 2 * wl.M * wl.K + 2 * used * wl.K * wl.N + 4 * wl.M + 2 * wl.M * wl.N
    sets = rotation_sets(nbytes)
    ws = [w] + [w.clone() for _ in range(sets - 1)]
    ys = [torch.empty((wl.M, wl.N), dtype=dtype, device="cuda") for _ in range(sets)]

    work = torch.empty(la.indexed_workspace_bytes(wl.E, wl.M), dtype=torch.uint8, device="cuda")

    def call(i):
        k = i % sets
        fn(x, ws[k], idx, out=ys[k], stream=stream, workspace=work)

    per_graph = graph_calls(sets)
    graph = capture(call, per_graph, stream, torch)
    replays = max(1, calls // per_graph)
    graph.replay()
    times = [time_region(graph, replays, stream, torch) for _ in range(5)]
    ms = sorted(times)[len(times) // 2] / (replays * per_graph)
    del graph, ws, ys
    return {"E": wl.E, "M": wl.M, "N": wl.N, "K": wl.K, "experts_used": used, "variant": dtype_name,
            "us_per_call": round(ms * 1e3, 3), "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 1),
            "hbm_gbs_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "input_sets": sets}


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_amd", "liblinear_probe.so"))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.probe_read.argtypes = [vp, i64, i32, vp, vp]
    lib.probe_empty.argtypes = [i32, vp]
    lib.probe_mfma.argtypes = [vp, i32, i32, vp, vp]
    lib.probe_loads.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    lib.probe_mfma_lds.argtypes = [vp, i32, i32, vp, vp]
    for f in (lib.probe_read, lib.probe_empty, lib.probe_mfma, lib.probe_loads, lib.probe_mfma_lds):
        f.restype = i32
    return lib


def bench_probe(kind, torch, workloads, stream):
    """Ceilings for the kernels' roofline fractions, measured with the probe
    kernels of liblinear_probe.so in graphs of 64 launches:
      read:  a plain read of the decode weight ([4096, 4096] binary16, 32 MiB),
             rotating over the same 16 copies as the decode benchmark, on the
             decode kernel's grid (256 workgroups of 512 threads);
      empty: an empty kernel on that grid (the per-launch floor);
      mfma:  register-only v_mfma_f32_32x32x16_f16 on random binary16 operands
             (1024 workgroups of 4 waves, 2000 rounds of 8 MFMAs per wave);
      mfma_lds: the attention projection's 512 tiles of 256 x 256 x 4096 with
             their fragments read from LDS (random binary16 data loaded into
             LDS once) and no operand loads from memory;
      loads_attn, loads_toy: the streaming GEMM's operand loads alone for the
             attention projection (256 x 256 tiles, 2 slots) and the toy layer
             (64 x 64 tiles, 4 slots), no fragment reads and no MFMAs, with the
             inputs rotating as in those shapes' own benchmarks."""
    lib = _probe_lib()
    sp = ctypes_stream(stream)
    if kind == "read":
        _, w, _ = workloads.workload_inputs("gemv1", seed=0, device="cuda")
        copies = rotation_sets(w.numel() * 2)
        ws = [w] + [w.clone() for _ in range(copies - 1)]
        sink = torch.zeros(256, dtype=torch.int32, device="cuda")
        nbytes = w.numel() * 2

        def call(i):
            rc = lib.probe_read(ws[i % copies].data_ptr(), nbytes, 256, sink.data_ptr(), sp)
            assert rc == 0, rc
        calls, per = graph_calls(copies), nbytes
    elif kind == "empty":
        def call(i):
            assert lib.probe_empty(256, sp) == 0
        calls, per = 64, 0
    elif kind == "mfma":
        g = torch.Generator(device="cpu").manual_seed(3)
        ops = torch.randn(4096 * 64 * 8, generator=g).to(torch.float16).to("cuda")
        grid, iters = 1024, 2000
        out = torch.empty(grid * 4 * 64 * 64, dtype=torch.float32, device="cuda")

        def call(i):
            assert lib.probe_mfma(ops.data_ptr(), grid, iters, out.data_ptr(), sp) == 0
        calls, per = 8, 0
    elif kind == "mfma_lds":
        g = torch.Generator(device="cpu").manual_seed(3)
        ops = torch.randn(4096 * 64 * 8, generator=g).to(torch.float16).to("cuda")
        grid, nk = 512, 64
        out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")

        def call(i):
            assert lib.probe_mfma_lds(ops.data_ptr(), grid, nk, out.data_ptr(), sp) == 0
        calls, per = 16, 0
    elif kind in ("loads_attn", "loads_toy"):
        name, tile, bm = ("attn", 0, 256) if kind == "loads_attn" else ("toy", 1, 64)
        wl = workloads.WORKLOADS[name]
        x, w, _ = workloads.workload_inputs(name, seed=0, device="cuda")
        sets = rotation_sets(wl.bytes)          # the same rotation as the layer's own benchmark
        xs = [x] + [x.clone() for _ in range(sets - 1)]
        ws = [w] + [w.clone() for _ in range(sets - 1)]
        tiles = (wl.M // bm) * (wl.N // bm)
        sink = torch.zeros(tiles, dtype=torch.int32, device="cuda")

        def call(i):
            rc = lib.probe_loads(xs[i % sets].data_ptr(), ws[i % sets].data_ptr(), wl.M, wl.N, wl.K, tile,
                                 sink.data_ptr(), sp)
            assert rc == 0, rc
        calls, per = graph_calls(sets), tiles * 2 * bm * wl.K * 2
    else:
        raise SystemExit("unknown probe %s" % kind)
    graph = capture(call, calls, stream, torch)
    graph.replay()
    replays = 4 if kind in ("mfma", "mfma_lds", "loads_attn") else max(1, 640 // calls)
    times = [time_region(graph, replays, stream, torch) for _ in range(5)]
    us = sorted(times)[2] / (replays * calls) * 1e3
    del graph
    torch.cuda.synchronize()
    r = {"probe": kind, "us_per_launch": round(us, 3)}
    if kind == "read":
        r.update({"bytes_per_launch": per, "gbs": round(per / (us * 1e-6) / 1e9, 1),
                  "frac_hbm_peak": round(per / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": copies})
    if kind.startswith("loads_"):
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        r.update({"name": name, "tile": [bm, bm], "input_sets": sets, "bytes_into_cus_per_launch": per,
                  "gbs_per_cu": round(per / cus / (us * 1e-6) / 1e9, 1)})
    if kind in ("mfma", "mfma_lds"):
        flops = grid * 4 * iters * 8 * 32768.0 if kind == "mfma" else grid * 8 * nk * 4 * 8 * 32768.0
        r.update({"flops_per_launch": flops, "tflops": round(flops / (us * 1e-6) / 1e12, 1),
                  "frac_mfma_peak": round(flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)})
    return r


def ctypes_stream(stream):
    return stream.cuda_stream if stream is not None else None


def cpu_baseline(workloads, target_s: float = 12.0):
    """The CPU oracle on the same decode step, repeated for ~target_s of wall time
    (a bounded sample of the workload; its rate is scaled to GB/s per step)."""
    import oracle
    orc = oracle.default()
    x1, w, b = workloads.workload_inputs("gemv1", seed=0)
    x16, _, _ = workloads.workload_inputs("gemv16", seed=0)
    step_bytes = workloads.WORKLOADS["gemv1"].bytes + workloads.WORKLOADS["gemv16"].bytes
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.linear(x1, w, b)
        orc.linear(x16, w, b)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 2000:
            break
    per_step = el / reps
    return {
        "value": round(step_bytes / per_step / 1e9, 3),
        "unit": "GB/s",
        "cores": orc.max_threads(),
        "kind": "oracle",
        "sample": "%d full decode steps (x[1,4096] and x[16,4096] against weight[4096,4096] + b), "
                  "%.1f s wall, %.1f ms per step" % (reps, el, per_step * 1e3),
        "ms_per_step": round(per_step * 1e3, 3),
    }


def cpu_baseline_gemm(name, workloads, target_s: float = 2.5):
    """The CPU oracle on one prefill shape, timed on a bounded sample: the first R
    rows of x against the whole weight and bias (R x N outputs, full K), R sized
    for about target_s of wall time (the toy runs whole).  Its rate is scaled to
    TFLOP/s of the full shape's 2MNK."""
    import oracle
    orc = oracle.default()
    wl = workloads.WORKLOADS[name]
    x, w, b = workloads.workload_inputs(name, seed=0)
    step = max(1, orc.max_threads())
    rows = min(wl.M, step)
    while True:
        # grow the sample until one call takes a quarter of the target, then size
        # the timed call from that rate
        t0 = time.perf_counter()
        orc.linear(x[:rows], w, b)
        el = time.perf_counter() - t0
        if rows == wl.M or el >= target_s / 4:
            break
        rows = min(wl.M, rows * 2)
    want = min(wl.M, max(rows, int(rows * target_s / max(el, 1e-9)) // step * step))
    if want != rows:
        rows = want
        t0 = time.perf_counter()
        orc.linear(x[:rows], w, b)
        el = time.perf_counter() - t0
    flops = 2.0 * rows * wl.N * wl.K
    return {
        "value": round(flops / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": orc.max_threads(),
        "kind": "oracle",
        "sample": "%d of %d rows of x against the full weight [%d, %d] and b, %.2f s wall%s"
                  % (rows, wl.M, wl.N, wl.K, el, " (the whole shape)" if rows == wl.M else ""),
        "full_shape_s_estimate": round(el * wl.M / rows, 2),
    }


def main():
    args = parse()
    if args.record_traffic:
        k, fd, wd, cfd, cwd = args.record_traffic
        record_traffic(k, fd, wd, cfd, cwd, [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py --only decode "
            "--steps 16 --warmup 8 --repeats 1",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py --only decode "
            "--steps 16 --warmup 8 --repeats 1",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <COPY_FETCH_DIR> -- python3 bench.py --only copycal",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <COPY_WRITE_DIR> -- python3 bench.py --only copycal",
        ])
        return
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs each call on one GPU and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_amd as la
    from linear_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    la._lib()
    stream = torch.cuda.Stream()
    log("device:", torch.cuda.get_device_name(0))

    if args.only:
        if args.only == "copycal":
            # a plain device-to-device copy of known size: the reference that scales the
            # FETCH_SIZE / WRITE_SIZE counters to bytes
            src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
            torch.cuda.synchronize()
            log("copycal: 5 copies of %d bytes" % (src.numel() * 4))
        elif args.only == "decode":
            dt = torch.bfloat16 if args.variant == "bf16" else torch.float16
            ms, _ = bench_decode(args, torch, la, workloads, stream, dt)
            log("decode ms/step %.5f" % ms)
        elif args.only.startswith("probe_"):
            log(json.dumps(bench_probe(args.only[len("probe_"):], torch, workloads, stream)))
        elif args.only == "context":
            log(json.dumps(bench_context(torch, la, workloads, stream)))
        elif args.only in workloads.GROUPED:
            log(json.dumps(bench_grouped(args.only, torch, la, workloads, stream, 40, args.variant)))
        elif args.only in workloads.INDEXED:
            log(json.dumps(bench_indexed(args.only, torch, la, workloads, stream, 200, args.variant)))
        else:
            log(json.dumps(bench_gemm(args.only, torch, la, workloads, stream, 100, args.variant)))
        return

    log("decode step: %d warmup, %d timed x %d repeats" % (args.warmup, args.steps, args.repeats))
    ms, detail = bench_decode(args, torch, la, workloads, stream)
    step_bytes = detail["step_bytes"]
    value = step_bytes / (ms * 1e-3) / 1e9
    launches = 2
    per_launch_bytes = step_bytes / launches
    per_launch_s = ms * 1e-3 / launches
    achieved = per_launch_bytes / per_launch_s / 1e9
    log("decode: %.3f us/step, %.1f GB/s" % (ms * 1e3, value))
    context = bench_context(torch, la, workloads, stream)
    for kind in ("read", "empty", "mfma", "mfma_lds"):
        log("probe", kind)
        context["probe_" + kind] = bench_probe(kind, torch, workloads, stream)
    # the decode launch's rate against a plain read of the same rotated weights on
    # its grid, measured in this run: the part's practical ceiling for this call
    context["decode_frac_of_probe_read"] = round(achieved / context["probe_read"]["gbs"], 4)
    log("context", json.dumps(context))

    prefill = {}
    if not args.no_prefill:
        for name, calls in (("toy", 400), ("attn", 50), ("mlp_up", 30), ("down", 50)):
            log("prefill", name)
            prefill[name] = bench_gemm(name, torch, la, workloads, stream, calls)
            log(json.dumps(prefill[name]))
        # the same calls' operand loads alone (probe kernels, same tiles, ring and
        # input rotation, no MFMAs): what share of each call the loads account for
        for kind, name in (("loads_toy", "toy"), ("loads_attn", "attn")):
            log("probe", kind)
            r = bench_probe(kind, torch, workloads, stream)
            r["frac_of_call"] = round(r["us_per_launch"] / prefill[name]["us_per_call"], 4)
            prefill[name]["operand_loads_alone"] = r
            log(json.dumps(r))
        # and attn's MFMAs with their fragments read from LDS, no operand loads
        # (the same 512 tiles of work): what share of the call the matrix work is
        m = dict(context["probe_mfma_lds"])
        m["frac_of_call"] = round(m["us_per_launch"] / prefill["attn"]["us_per_call"], 4)
        prefill["attn"]["mfma_fed_from_lds_alone"] = m
    variants = {}
    if not args.no_variants:
        dargs = argparse.Namespace(steps=args.steps, warmup=args.warmup, repeats=args.repeats)
        dms, _ = bench_decode(dargs, torch, la, workloads, stream, torch.bfloat16)
        variants["decode_bf16"] = {"us_per_step": round(dms * 1e3, 3),
                                   "gbs": round(step_bytes / (dms * 1e-3) / 1e9, 1),
                                   "frac_hbm_peak": round(step_bytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log("decode bf16", json.dumps(variants["decode_bf16"]))
        if not args.no_prefill:
            for name, calls, var in (("attn", 50, "bf16"), ("attn", 50, "f16_f32out"),
                                     ("attn", 50, "bf16_f32out"), ("down", 50, "bf16"),
                                     ("mlp_up", 30, "f16_epi_gelu"), ("down", 50, "f16_epi_res"),
                                     ("attn", 50, "f16_epi_silu_mul"), ("gemv16", 400, "f16_epi_silu")):
                variants["%s_%s" % (name, var)] = r = bench_gemm(name, torch, la, workloads, stream, calls, var)
                log(json.dumps(r))
            variants["grouped_f16"] = r = bench_grouped("grouped", torch, la, workloads, stream, 40)
            log(json.dumps(r))
            for name, calls in (("moe_decode", 400), ("moe_prefill", 40)):
                variants["%s_f16" % name] = r = bench_indexed(name, torch, la, workloads, stream, calls)
                log(json.dumps(r))
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(workloads)
        log(json.dumps(cpu))
        for name in prefill:
            prefill[name]["cpu_baseline"] = r = cpu_baseline_gemm(name, workloads)
            log(name, json.dumps(r))

    line = {
        "metric": "TFLOP/s and % FP16 MFMA peak (large M); HBM GB/s and % peak (M≤16)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded: x~N(0,1), weight,b~U(-1/64,1/64))",
        "config": {
            "workload": "decode GEMV batch: y=FP16(FP16(x@W.T)+b), x [1,4096] and [16,4096], "
                        "W [4096,4096], b [4096], fp16",
            "accumulate": "f32 (products exact, FP32 sums rounded once to f16 before the bias)",
            "calls_per_step": launches,
            "weight_copies_rotated": detail["weight_copies"],
            "steps_per_graph": detail["steps_per_graph"],
            "timed_as": "%d replays of the %d-step graph + one %d-step graph, between two events, "
                        "device synchronised on both sides" % (detail["graph_replays"]["full"],
                                                               detail["steps_per_graph"],
                                                               detail["graph_replays"]["remainder_steps"]),
            "warmup_as": "%d steps replayed through the same graphs (plus %d steps run eagerly while "
                         "capturing them)" % (args.warmup, detail["eager_steps_at_capture"]),
            "kernel": "M = 1: gemv_stream<f16, bias> (one wave per weight row, 4 rows per workgroup, FP32 "
                      "FMAs); M = 16: skinny_stream<8, f16, bias> (16 output columns x 16 rows per workgroup, "
                      "8 waves, v_mfma_f32_16x16x32_f16)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("decode_f16_step"),
            "kernel": "decode_f16_step: gemv_stream (M = 1) and skinny_stream (M = 16), one launch each",
            "bytes_per_launch": per_launch_bytes,
            "us_per_launch": round(per_launch_s * 1e6, 3),
        },
        "cpu_baseline": cpu,
        "context": context,
        "prefill": prefill,
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
