#!/usr/bin/env python3
"""Benchmark of the fused add + argmax readout on one MI355X.

One step = one call of ``xpress_add_argmax_to_blk`` over a whole batch of
draft rows (every stage of the readout: stream loads, add + bf16 rounding,
the (value, index) reduction, the cross-workgroup combine and the scatter
into blk).  Inputs are resident in HBM before the timed region starts; the
call rotates over several identical copies of the inputs whose total size
exceeds twice the 256 MB last-level cache, so each call streams from HBM.

Prints ONE JSON line.  ``value`` is effective HBM GB/s = rows * V * 4 bytes
(two bf16 streams) per call over the wall time of the timed calls.
``roofline.achieved`` uses the same algorithmic bytes over the average
readout-kernel duration measured with HIP events on the launch stream.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same rows
on the host cores, and the GPU's answers for those rows are checked against
it.

The default warmup (300 steps, ~14 ms) covers the clock ramp measured on
MI355X: under sustained back-to-back calls the readout settles after about
200 calls.

``--op topc --topc-c C`` times the top-C readout (``xpress_topc_argmax_to_blk``)
on the synthetic top-C workload with C candidates per row instead; the
default is the full-vocabulary readout.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--op readout|topc] [--topc-c C]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
LLC_BYTES = 256 * 2 ** 20    # MI355X Infinity Cache
CSRC = os.path.join(ROOT, "vocab_wide_add_amd", "csrc")
_COMMON = [os.path.join(CSRC, "device_common.h"), os.path.join(CSRC, "host_common.h"),
           os.path.join(ROOT, "include", "xpress_argmax.h")]
# every source a kernel's code is compiled from (the readout with in-place
# bias also runs the key reduction of xpress_argmax.hip)
SRC = [os.path.join(CSRC, "xpress_argmax.hip")] + _COMMON
GEMM_SRC = [os.path.join(CSRC, "readout_gemm.hip"), os.path.join(CSRC, "xpress_argmax.hip")] + _COMMON


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def source_digest(src=SRC) -> str:
    """SHA-256 of the code of every source a kernel is compiled from (a path
    or a list of paths): comments removed and whitespace runs collapsed, so
    that counters recorded for the code stay valid across edits of its
    comments and are dropped by any change to the code itself."""
    paths = [src] if isinstance(src, str) else list(src)
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode() + b"\0")
    return h.hexdigest()


def traffic_for(workload: str, src: str = SRC):
    """HBM bytes per launch from committed PMC counter runs, if they were
    taken on the current source of the kernel (src); else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_digest(src):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model string (/proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_cores() -> int:
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(cores or 1, 64))


def cpu_baseline(base, bias, w, target_s: float):
    """The oracle, as is, on the host cores: three timed runs on all cores
    (rows spread over threads) and three on one thread, each run as many
    whole passes over its sample of rows as fit in about target_s / 6
    seconds; the medians are reported.  Returns (result dict, rows checked,
    the oracle's answers for those rows)."""
    import statistics
    import oracle
    cores = host_cores()
    per_run = max(0.2, target_s / 6.0)
    t0 = time.perf_counter()
    oracle.add_argmax_rows(base, bias, 0, 1, w.V, w.stride_base, w.stride_bias)
    t_row = max(time.perf_counter() - t0, 1e-4)

    def runs(rows, threads):
        rates, ans = [], None
        for _ in range(3):
            passes, t0 = 0, time.perf_counter()
            while True:
                if threads > 1:
                    ans = oracle.add_argmax_rows_threaded(base, bias, rows, w.V, w.stride_base,
                                                          w.stride_bias, threads)
                else:
                    ans = oracle.add_argmax_rows(base, bias, 0, rows, w.V, w.stride_base,
                                                 w.stride_bias)
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= per_run or passes >= 1000:
                    break
            rates.append(passes * rows / dt)
        return rates, ans

    rows_mc = int(min(w.rows, max(cores, per_run * cores / t_row)))
    rows_st = int(min(w.rows, max(1, per_run / t_row)))
    mc, ans = runs(rows_mc, cores)
    st, _ = runs(rows_st, 1)
    gbs = lambda r: round(r * w.V * 4 / 1e9, 3)
    res = {"value": gbs(statistics.median(mc)), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "rows_per_s": round(statistics.median(mc), 1),
           "runs": [gbs(r) for r in mc],
           "cpu_model": cpu_model(),
           "single_thread": {"value": gbs(statistics.median(st)), "unit": "GB/s",
                             "rows_per_s": round(statistics.median(st), 1),
                             "runs": [gbs(r) for r in st],
                             "sample": "first %d rows of %s" % (rows_st, w.name)},
           "sample": "first %d of %d rows of %s; median of 3 runs of ~%.1f s each on %d threads "
                     "(and 3 on one thread)" % (rows_mc, w.rows, w.name, per_run, cores)}
    return res, rows_mc, ans


def copy_probe(nbytes: int, reps: int):
    """A plain device-to-device copy of known size (for scaling PMC counters)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def time_graph(step, steps: int, warmup: int, per_graph: int, reserve):
    """Capture ``per_graph`` steps into one HIP graph and time ``steps``
    steps as graph replays (region 1: wall clock and one HIP event pair
    around the replays).  Returns (wall seconds, GPU seconds, steps replayed)."""
    import torch
    cap = torch.cuda.Stream()
    reserve(cap)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for k in range(per_graph):
            step(k, cap)
    reps = max(1, steps // per_graph)
    for _ in range(max(1, warmup // per_graph)):
        graph.replay()
    torch.cuda.synchronize()
    log("timing %d graph replays of %d steps" % (reps, per_graph))
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(cur)
    for _ in range(reps):
        graph.replay()
    r1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, r0.elapsed_time(r1) * 1e-3, reps * per_graph


def read_ceiling(native, dev, w, sets: int, stream, reps: int):
    """The plain two-stream read of the same inputs (xpress_read_probe), one
    workgroup per row and grid-stride, each timed over `reps` launches with
    HIP events on the launch stream after 50 untimed ones.  None when the
    layout is not one the probe reads (equal, 8-element-aligned strides)."""
    import torch
    if w.V % 8 or w.stride_base != w.stride_bias or w.stride_base % 8:
        return None
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for mode, name in ((native.XPRESS_READ_ROWS, "per_row"),
                       (native.XPRESS_READ_FLAT, "grid_stride")):
        def probe(k):
            b, i = dev[k % sets][0], dev[k % sets][1]
            native.xpress_read_probe(b, i, w.rows, w.V, w.stride_base, mode, sink, stream=stream)
        for k in range(50):
            probe(k)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(reps):
            probe(k)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = w.bytes_read if mode == native.XPRESS_READ_ROWS else \
            ((w.rows - 1) * w.stride_base + w.V) * 4
        out[name] = {"us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1), "bytes": nbytes,
                     "launches": reps}
    return out


def last_set(args, sets: int) -> int:
    """Input set written by the last timed step: step k uses set k % sets; a
    captured graph replays steps 0 .. per_graph - 1."""
    last = (args.graph if args.graph else args.steps) - 1
    return last % sets


def time_steps(step, steps: int, warmup: int, stream):
    """Warm up, then time ``steps`` calls twice: region 1 back to back (wall
    clock and one HIP event pair on the launch stream around the region),
    region 2 with a HIP event pair around every call.  Returns (wall seconds
    of region 1, GPU seconds of region 1, sorted per-call GPU seconds of
    region 2)."""
    import torch
    log("warming up: %d steps" % warmup)
    # the events exist (and have been recorded once) before the timed region,
    # so that no event creation lands inside it
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    r1.record(stream)
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    log("timing %d steps" % steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for k in range(steps):
        step(k)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_gpu = r0.elapsed_time(r1) * 1e-3
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        starts[k].record(stream)
        step(k)
        ends[k].record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) * 1e-3 for a, b in zip(starts, ends))
    return wall, region_gpu, durs


def result_line(metric, name, config, bytes_per_call, rows, steps, warmup, wall, region_gpu,
                durs, launches, traffic):
    kavg = sum(durs) / len(durs)
    # the kernel's average duration: GPU time of timed region 1 (HIP events
    # on the launch stream) per launch.  The default workload's plan is one
    # launch per step; the per-launch event pairs of region 2 carry ~2 us of
    # event overhead each and are reported beside it.
    kernel_avg = region_gpu / steps / max(1, launches)
    achieved = bytes_per_call / max(1, launches) / kernel_avg / 1e9
    value = bytes_per_call * steps / wall / 1e9
    return {
        "metric": metric,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(rows * steps / wall, 1),
        "region_gpu_us_per_step": round(region_gpu / steps * 1e6, 3),
        "kernel_us_region_avg": round(kernel_avg * 1e6, 3),
        "kernel_us_event_pairs": {"avg": round(kavg * 1e6, 3), "min": round(durs[0] * 1e6, 3),
                                  "p10": round(durs[int(len(durs) * 0.1)] * 1e6, 3),
                                  "p50": round(durs[len(durs) // 2] * 1e6, 3),
                                  "p90": round(durs[int(len(durs) * 0.9)] * 1e6, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "traffic_source": ("committed counter record profiles/traffic_%s.json (rocprofv3 "
                           "FETCH_SIZE and WRITE_SIZE per launch, scaled by a 1 GiB copy's "
                           "counters), taken on this kernel source (digest matched); not "
                           "measured in this run" % name) if traffic is not None else
                          "no counter record for this kernel source",
        "cpu_baseline": None,
    }


def bench_readout(args, np, torch, native, workloads):
    name = args.workload or workloads.BENCH_WORKLOAD
    w = workloads.WORKLOADS[name]
    log("generating %s" % name)
    base, bias, blk0 = workloads.generate(w)
    footprint = base.nbytes + bias.nbytes
    sets = max(1, math.ceil(2 * LLC_BYTES / footprint) + 1)
    log("uploading %d input sets of %.1f MB" % (sets, footprint / 1e6))
    b_cpu = torch.from_numpy(base.view(np.int16))
    i_cpu = torch.from_numpy(bias.view(np.int16))
    dev = [(b_cpu.cuda(), i_cpu.cuda(), torch.from_numpy(blk0).cuda()) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    plan = native.xpress_describe_plan(dev[0][0], dev[0][1], w.N, w.B, w.V,
                                       w.stride_base, w.stride_bias)
    native.xpress_reserve(w.N, w.B, w.V, stream=stream)

    # the binding's checks (tensor spans, stream lookup) once per input set
    # here; each timed step is then one call of the C entry point, which
    # validates its arguments itself
    calls = [native.bind_add_argmax_to_blk(b, i, blk, w.N, w.B, w.V, w.stride_base,
                                           w.stride_bias, stream=stream) for b, i, blk in dev]

    def step(k, st=stream):
        if st is stream:
            calls[k % sets]()
            return
        b, i, blk = dev[k % sets]
        native.xpress_add_argmax_to_blk(b, i, blk, w.N, w.B, w.V, w.stride_base,
                                        w.stride_bias, stream=st)

    if args.graph:
        wall, region_gpu, n = time_graph(step, args.steps, args.warmup, args.graph,
                                         lambda st: native.xpress_reserve(w.N, w.B, w.V, stream=st))
        args.steps = n
        durs = [region_gpu / n]
    else:
        wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    got = dev[last_set(args, sets)][2].cpu().numpy()
    config = {"workload": name, "N": w.N, "B": w.B, "V": w.V, "rows": w.rows,
              "stride_base": w.stride_base, "stride_bias": w.stride_bias,
              "bytes_per_step": w.bytes_read, "input_sets": sets, "plan": plan,
              "launch": ("hip graph of %d steps" % args.graph) if args.graph else "stream"}
    out = result_line("effective HBM GB/s (+ %% of peak) and rows/s, add+argmax N=%d B=%d V=%d"
                      % (w.N, w.B, w.V), name, config, w.bytes_read, w.rows, args.steps,
                      args.warmup, wall, region_gpu, durs, plan["launches"], traffic_for(name))
    if not args.graph and not args.no_graph_form:
        # context beside the stream figure: the same steps captured in a HIP
        # graph (the deployment form of a pass), after the timed regions
        log("graph form")
        per_graph = min(args.steps, 50)
        g_wall, g_gpu, g_n = time_graph(step, args.steps, per_graph, per_graph,
                                        lambda st: native.xpress_reserve(w.N, w.B, w.V, stream=st))
        out["graph_form"] = {"launch": "hip graph of %d steps" % per_graph, "steps": g_n,
                             "us_per_step_wall": round(g_wall / g_n * 1e6, 3),
                             "us_per_step_gpu": round(g_gpu / g_n * 1e6, 3),
                             "GBps_wall": round(w.bytes_read * g_n / g_wall / 1e9, 1)}
    if not args.no_read_ceiling:
        log("read ceiling")
        rc = read_ceiling(native, dev, w, sets, stream, max(200, min(args.steps, 1000)))
        if rc is not None:
            k_us = out["kernel_us_region_avg"]
            rc["readout_over_per_row"] = round(rc["per_row"]["us"] / k_us, 4)
            rc["readout_over_grid_stride"] = round(rc["grid_stride"]["us"] / k_us, 4)
        out["read_ceiling"] = rc
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cb, nrows, ans = cpu_baseline(base, bias, w, args.cpu_seconds)
        out["cpu_baseline"] = cb
        out["checked_rows"] = nrows
        out["checked_equal"] = bool(np.array_equal(got[:, 1:].reshape(-1)[:nrows], ans))
        if not out["checked_equal"]:
            log("MISMATCH against the oracle on the sampled rows")
    return out


def bench_read(args, np, torch, native, workloads):
    """The read ceiling alone as the timed step: xpress_read_probe over the
    readout's inputs (--read-mode rows: one workgroup per row; flat:
    grid-stride), for profiling it under the same command shape."""
    name = args.workload or workloads.BENCH_WORKLOAD
    w = workloads.WORKLOADS[name]
    if w.V % 8 or w.stride_base != w.stride_bias or w.stride_base % 8:
        raise SystemExit("the read probe needs equal, 8-element-aligned strides")
    log("generating %s" % name)
    base, bias, blk0 = workloads.generate(w)
    footprint = base.nbytes + bias.nbytes
    sets = max(1, math.ceil(2 * LLC_BYTES / footprint) + 1)
    b_cpu = torch.from_numpy(base.view(np.int16))
    i_cpu = torch.from_numpy(bias.view(np.int16))
    dev = [(b_cpu.cuda(), i_cpu.cuda()) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    mode = native.XPRESS_READ_ROWS if args.read_mode == "rows" else native.XPRESS_READ_FLAT
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = w.bytes_read if mode == native.XPRESS_READ_ROWS else \
        ((w.rows - 1) * w.stride_base + w.V) * 4

    def step(k, st=stream):
        b, i = dev[k % sets]
        native.xpress_read_probe(b, i, w.rows, w.V, w.stride_base, mode, sink, stream=st)

    wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    config = {"workload": name, "op": "read", "mode": args.read_mode, "rows": w.rows, "V": w.V,
              "bytes_per_step": nbytes, "input_sets": sets, "launch": "stream"}
    return result_line("plain streaming read of the readout's inputs (%s): effective GB/s"
                       % args.read_mode, name, config, nbytes, w.rows, args.steps, args.warmup,
                       wall, region_gpu, durs, 1, None)


def bench_topc(args, np, torch, native, workloads):
    name = "topc_n32_b16_c%d" % args.topc_c
    w = workloads.TOPC_WORKLOADS[name]
    log("generating %s" % name)
    base_c, bias_c, cand, blk0 = workloads.generate_topc(w)
    footprint = base_c.nbytes + bias_c.nbytes + cand.nbytes
    # the inputs are small; rotate over enough copies to leave the 256 MB
    # last-level cache, capped at 64 copies
    sets = int(min(64, max(1, math.ceil(2 * LLC_BYTES / footprint) + 1)))
    log("uploading %d input sets of %.2f MB" % (sets, footprint / 1e6))
    b_cpu = torch.from_numpy(base_c.view(np.int16))
    i_cpu = torch.from_numpy(bias_c.view(np.int16))
    c_cpu = torch.from_numpy(cand)
    dev = [(b_cpu.cuda(), i_cpu.cuda(), c_cpu.cuda(), torch.from_numpy(blk0).cuda())
           for _ in range(sets)]
    stream = torch.cuda.current_stream()
    plan = native.xpress_describe_plan(dev[0][0], dev[0][1], w.N, w.B, w.C, w.C, w.C)
    native.xpress_reserve(w.N, w.B, w.C, stream=stream)

    def step(k, st=stream):
        b, i, c, blk = dev[k % sets]
        native.xpress_topc_argmax_to_blk(b, i, c, blk, w.N, w.B, w.C, stream=st)

    if args.graph:
        wall, region_gpu, n = time_graph(step, args.steps, args.warmup, args.graph,
                                         lambda st: native.xpress_reserve(w.N, w.B, w.C, stream=st))
        args.steps = n
        durs = [region_gpu / n]
    else:
        wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    config = {"workload": name, "op": "topc", "N": w.N, "B": w.B, "C": w.C, "rows": w.rows,
              "bytes_per_step": w.bytes_read, "input_sets": sets, "plan": plan,
              "launch": ("hip graph of %d steps" % args.graph) if args.graph else "stream"}
    out = result_line("top-C readout: effective GB/s and rows/s, N=%d B=%d C=%d"
                      % (w.N, w.B, w.C), name, config, w.bytes_read, w.rows, args.steps,
                      args.warmup, wall, region_gpu, durs, plan["launches"], None)
    got = dev[last_set(args, sets)][3].cpu().numpy()
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline")
        passes, t0 = 0, time.perf_counter()
        while True:
            want = blk0.copy()
            oracle.topc_argmax_to_blk(base_c, bias_c, cand, want, w.N, w.B, w.C)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min(args.cpu_seconds, 5.0) or passes >= 1000:
                break
        out["cpu_baseline"] = {"value": round(passes * w.bytes_read / dt / 1e9, 3),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "rows_per_s": round(passes * w.rows / dt, 1),
                               "sample": "all %d rows of %s, %d passes, %.1f s, one thread"
                                         % (w.rows, name, passes, dt)}
        out["checked_rows"] = w.rows
        out["checked_equal"] = bool(np.array_equal(got, want))
    return out


def bench_gemm(args, np, torch, native, workloads):
    name = args.workload if (args.workload or "").startswith("gemm_") else workloads.GEMM_BENCH_WORKLOAD
    w = workloads.GEMM_WORKLOADS[name]
    log("generating %s" % name)
    base, x, wt, blk0 = workloads.generate_gemm(w)
    footprint = base.nbytes + x.nbytes + wt.nbytes
    sets = max(1, math.ceil(2 * LLC_BYTES / footprint) + 1)
    log("uploading %d input sets of %.1f MB" % (sets, footprint / 1e6))
    cpu = [torch.from_numpy(t.view(np.int16)) for t in (base, x, wt)]
    dev = [tuple(t.cuda() for t in cpu) + (torch.from_numpy(blk0).cuda(),) for _ in range(sets)]
    stream = torch.cuda.current_stream()

    def step(k, st=stream):
        b, xx, ww, blk = dev[k % sets]
        native.xpress_readout_gemm_argmax_to_blk(b, xx, ww, blk, w.N, w.B, w.V, w.R, w.V,
                                                 stream=st)

    wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    # the fused path's answers, before the unfused context path reuses blk
    got = dev[last_set(args, sets)][3].cpu().numpy()[:, 1:].reshape(-1)
    config = {"workload": name, "op": "readout_gemm", "N": w.N, "B": w.B, "V": w.V, "R": w.R,
              "rows": w.rows, "bytes_per_step": w.bytes_read, "flops_per_step": w.flops,
              "input_sets": sets, "launches_per_step": 2}
    out = result_line("readout with in-place bias (x @ w.T): effective GB/s and rows/s, "
                      "N=%d B=%d V=%d R=%d" % (w.N, w.B, w.V, w.R), name, config, w.bytes_read,
                      w.rows, args.steps, args.warmup, wall, region_gpu, durs, 2,
                      traffic_for(name, GEMM_SRC))
    out["tflops"] = round(w.flops * args.steps / wall / 1e12, 2)
    out["roofline"]["note"] = ("two launches per pass (the fused kernel and the key "
                               "reduction); achieved is over the pass's GPU time, and "
                               "kernel_us_region_avg is that time over both launches")

    # context: the unfused path -- a library matmul writing the bf16 bias,
    # then this library's readout over base and that bias
    # (the weight is transposed once into a contiguous [R, V] copy: the library
    # matmul then sees no transposed view)
    bias = [torch.empty((w.rows, w.V), dtype=torch.bfloat16, device="cuda")]
    w_t = [d[2].view(torch.bfloat16).t().contiguous() for d in dev]

    def unfused(k, st=stream):
        b, xx, ww, blk = dev[k % sets]
        torch.matmul(xx.view(torch.bfloat16), w_t[k % sets], out=bias[0])
        native.xpress_add_argmax_to_blk(b, bias[0].view(torch.int16), blk, w.N, w.B, w.V, w.V,
                                        w.V, stream=st)

    uw, ug, _ = time_steps(unfused, max(50, args.steps // 5), max(20, args.warmup // 5), stream)
    out["unfused_us_per_step"] = round(ug / max(50, args.steps // 5) * 1e6, 2)
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline")
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1
        n = max(cores, 16)
        rows = list(range(0, w.rows, max(1, w.rows // n)))[:n]
        t0 = time.perf_counter()
        ans = oracle.gemm_argmax_rows(base, x, wt, rows, w.V, w.R, w.V, threads=cores)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(len(rows) * (w.V * 2 + w.R * 2) / dt / 1e9, 4),
                               "unit": "GB/s", "cores": cores, "kind": "oracle",
                               "rows_per_s": round(len(rows) / dt, 2),
                               "sample": "%d of %d rows of %s, %.1f s on %d threads"
                                         % (len(rows), w.rows, name, dt, cores)}
        out["checked_rows"] = len(rows)
        out["checked_equal_rows"] = int(np.sum(got[rows] == ans))
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def bench_latent(args, np, torch, native, workloads):
    name = args.workload if (args.workload or "").startswith("latent_") else \
        workloads.LATENT_BENCH_WORKLOAD
    w = workloads.LATENT_WORKLOADS[name]
    log("generating %s" % name)
    d = workloads.generate_latent(w)
    keys = ("blk", "am1", "xh", "w1", "wlat", "mixl", "wg", "wu", "wd")
    dev = {k: torch.from_numpy(d[k].view(np.int16) if d[k].dtype == np.uint16 else d[k]).cuda()
           for k in keys}
    out_d = torch.empty((w.N, w.B - 1, w.R), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    native.xpress_latent_reserve(w.N, w.B, w.R, w.H, stream=stream)
    tiles = tuple(int(t) for t in args.latent_tiles.split(","))
    native.xpress_latent_set_tiles(*tiles)

    def step(k, st=stream):
        native.xpress_latent_pass(*(dev[x] for x in keys), out_d, w.N, w.B, w.R, w.H, w.V,
                                  stream=st)

    if args.graph:
        wall, region_gpu, n = time_graph(
            step, args.steps, args.warmup, args.graph,
            lambda st: native.xpress_latent_reserve(w.N, w.B, w.R, w.H, stream=st))
        args.steps = n
        durs = [region_gpu / n]
    else:
        wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    got = out_d.cpu().numpy().view(np.uint16)
    per_pass = region_gpu / args.steps
    achieved = w.flops / per_pass / 1e12
    out = {
        "metric": "latent stage of one pass: blocks/s and us per pass, N=%d B=%d R=%d H=%d"
                  % (w.N, w.B, w.R, w.H),
        "value": round(w.N * args.steps / wall, 1),
        "unit": "blocks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "op": "latent", "N": w.N, "B": w.B, "R": w.R, "H": w.H,
                   "V": w.V, "flops_per_step": w.flops, "bytes_per_step": w.bytes_moved,
                   "launches_per_step": 3, "tiles": args.latent_tiles,
                   "caches": "one input set: the ~1 MB of weights stay cache-resident",
                   "launch": ("hip graph of %d steps" % args.graph) if args.graph else "stream"},
        "us_per_pass": round(per_pass * 1e6, 3),
        "pass_us_event_pairs": {"avg": round(sum(durs) / len(durs) * 1e6, 3),
                                "min": round(durs[0] * 1e6, 3),
                                "p10": round(durs[int(len(durs) * 0.1)] * 1e6, 3),
                                "p50": round(durs[len(durs) // 2] * 1e6, 3),
                                "p90": round(durs[int(len(durs) * 0.9)] * 1e6, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 5), "traffic": None,
                     "note": "three kernels per pass; achieved over the pass's GPU time"},
        "cpu_baseline": None,
    }

    # context: the same stage as separate torch operations (gather, matmuls,
    # mixer, SwiGLU), each its own launch
    f32 = {k: dev[k].view(torch.bfloat16).float() for k in ("xh", "mixl")}
    wb = {k: dev[k].view(torch.bfloat16) for k in ("w1", "wlat", "wg", "wu", "wd")}
    wt = {k: wb[k].t().contiguous() for k in ("wlat", "wg", "wu", "wd")}
    toks = torch.cat([dev["am1"].view(-1, 1), dev["blk"][:, :w.B - 1]], dim=1)

    def torch_stage(k, st=stream):
        emb = wb["w1"].index_select(0, toks.reshape(-1))
        x = f32["xh"] + torch.matmul(emb, wt["wlat"]).float().view(w.N, w.B, w.R)
        u = (f32["mixl"].unsqueeze(0) * x.unsqueeze(1)).sum(dim=2)[:, 1:].reshape(-1, w.R)
        ub = u.to(torch.bfloat16)
        g = torch.matmul(ub, wt["wg"]).float()
        v = torch.matmul(ub, wt["wu"]).float()
        m = (torch.nn.functional.silu(g) * v).to(torch.bfloat16)
        return (u + torch.matmul(m, wt["wd"]).float()).to(torch.bfloat16)

    tw, tg, _ = time_steps(torch_stage, max(50, args.steps // 5), max(20, args.warmup // 5),
                           stream)
    out["torch_ops_us_per_pass"] = round(tg / max(50, args.steps // 5) * 1e6, 2)
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline")
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1
        passes, t0 = 0, time.perf_counter()
        while True:
            want = oracle.latent_pass(*(d[x] for x in keys), w.N, w.B, w.R, w.H, w.V,
                                      threads=cores)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= args.cpu_seconds or passes >= 1000:
                break
        out["cpu_baseline"] = {"value": round(passes * w.N / dt, 2), "unit": "blocks/s",
                               "cores": cores, "kind": "oracle",
                               "us_per_pass": round(dt / passes * 1e6, 1),
                               "sample": "all %d blocks of %s, %d passes, %.1f s on %d threads"
                                         % (w.N, name, passes, dt, cores)}
        out["checked_equal_fraction"] = round(float(np.mean(got == want)), 5)
    return out


def bench_pass(args, np, torch, native, workloads):
    """One whole pass: the latent stage (reading blk) feeding the readout
    with in-place bias (writing blk in place), back to back on one stream."""
    name = args.workload if (args.workload or "").startswith("pass_") else \
        workloads.PASS_BENCH_WORKLOAD
    lname, gname = workloads.PASS_WORKLOADS[name]
    lw, gw = workloads.LATENT_WORKLOADS[lname], workloads.GEMM_WORKLOADS[gname]
    assert (lw.N, lw.B, lw.R, lw.V) == (gw.N, gw.B, gw.R, gw.V)
    N, B, R, H, V = lw.N, lw.B, lw.R, lw.H, lw.V
    log("generating %s (%s + %s)" % (name, lname, gname))
    d = workloads.generate_latent(lw)
    base, _, wt, _ = workloads.generate_gemm(gw)
    keys = ("blk", "am1", "xh", "w1", "wlat", "mixl", "wg", "wu", "wd")
    dev = {k: torch.from_numpy(d[k].view(np.int16) if d[k].dtype == np.uint16 else d[k]).cuda()
           for k in keys}
    base_d = torch.from_numpy(base.view(np.int16)).cuda()
    wt_d = torch.from_numpy(wt.view(np.int16)).cuda()
    lat = torch.empty((N, B - 1, R), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(k, st=stream):
        native.xpress_latent_pass(*(dev[x] for x in keys), lat, N, B, R, H, V, stream=st)
        native.xpress_readout_gemm_argmax_to_blk(base_d, lat, wt_d, dev["blk"], N, B, V, R, V,
                                                 stream=st)

    def reserve(st):
        # both entry points share the stream's workspace: size it outside
        # capture with one eager pass on that stream
        native.xpress_latent_reserve(N, B, R, H, stream=st)
        step(0, st)
        torch.cuda.synchronize()

    reserve(stream)
    if args.graph:
        wall, region_gpu, n = time_graph(step, args.steps, args.warmup, args.graph, reserve)
        args.steps = n
        durs = [region_gpu / n]
    else:
        wall, region_gpu, durs = time_steps(step, args.steps, args.warmup, stream)
    per_pass = region_gpu / args.steps
    nbytes = lw.bytes_moved + gw.bytes_read
    flops = lw.flops + gw.flops
    achieved = nbytes / per_pass / 1e9
    blk = dev["blk"].cpu().numpy()
    return {
        "metric": "one pass (latent stage + readout with in-place bias): passes/s and us per "
                  "pass, N=%d B=%d R=%d H=%d V=%d" % (N, B, R, H, V),
        "value": round(args.steps / wall, 1),
        "unit": "passes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "op": "pass", "latent": lname, "readout": gname,
                   "N": N, "B": B, "R": R, "H": H, "V": V, "bytes_per_step": nbytes,
                   "flops_per_step": flops, "launches_per_step": 5,
                   "launch": ("hip graph of %d steps" % args.graph) if args.graph else "stream"},
        "us_per_pass": round(per_pass * 1e6, 3),
        "tflops": round(flops / per_pass / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "note": "five kernels per pass; achieved over the pass's GPU time"},
        "cpu_baseline": None,
        "blk_in_range": bool(((blk[:, 1:] >= 0) & (blk[:, 1:] < V)).all()),
        "anchor_kept": bool(np.array_equal(blk[:, 0], d["blk"][:, 0])),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--op", choices=["readout", "topc", "gemm", "latent", "pass", "read"],
                    default="readout")
    ap.add_argument("--read-mode", choices=["rows", "flat"], default="rows",
                    help="--op read: one workgroup per row, or grid-stride")
    ap.add_argument("--no-graph-form", action="store_true",
                    help="readout: skip the graph-form context figure")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the read-ceiling leg of the readout line")
    ap.add_argument("--graph", type=int, default=0,
                    help="capture this many steps per HIP graph and time graph replays")
    ap.add_argument("--topc-c", type=int, default=1024, choices=[64, 256, 1024, 4096])
    ap.add_argument("--latent-tiles", default="0,0,0",
                    help="row-slab counts of the mix, gate and down kernels (0 = automatic)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work budget of the oracle baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="only run a plain copy of this many bytes (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the readout has no cross-GPU step, and rows "
              "shard across GPUs with no exchange; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from vocab_wide_add_amd import native, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_bytes:
        copy_probe(args.copy_probe_bytes, max(1, args.steps))
        return
    if args.op == "topc":
        out = bench_topc(args, np, torch, native, workloads)
    elif args.op == "gemm":
        out = bench_gemm(args, np, torch, native, workloads)
    elif args.op == "latent":
        out = bench_latent(args, np, torch, native, workloads)
    elif args.op == "pass":
        out = bench_pass(args, np, torch, native, workloads)
    elif args.op == "read":
        out = bench_read(args, np, torch, native, workloads)
    else:
        out = bench_readout(args, np, torch, native, workloads)
    print(json.dumps(out))
    sys.stdout.flush()


if __name__ == "__main__":
    main()
