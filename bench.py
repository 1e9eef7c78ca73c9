"""Benchmark of the TQ2_0_g128 ternary GEMM (and the binary low-rank forward) on one MI355X.

Headline: weight-GB/s of tq2_gemm at M=1 (decode GEMV, N=K=4096), i.e. packed
weight bytes (N*K/128*34) per call over the per-call time.  A decode step is one
pass over L = 121 separately uploaded weights of that shape (a 121-layer decode:
more weight bytes than twice the 256 MB Infinity Cache), so every call streams
its weight from HBM whatever the step count.  The same JSON line also reports
the M=2048 prefill TFLOP/s, the small-batch MLP up-projection (steps of 35
weights), the two DiT benchmark shapes and the BLR layer forward and backward,
each with its roofline fraction, the launch and HBM floors of the box, and the
CPU oracle timed on this host's cores on bounded samples.

Timing: W untimed warmup steps, then exactly K steps between two device
synchronisations.  The K steps are captured once in a HIP graph and replayed, so
the timed region holds GPU work only (host launch cost removed); HIP events on
the launch stream bracket each replay, and the per-step time is the median
replay / K.  The same K steps issued eagerly from Python are also timed and
reported as context.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only decode,prefill,mlp,dit,blr,dense,cpu]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense f16 MFMA
F32_VALU_PEAK_TFLOPS = 157.3   # fp32 vector
MALL_BYTES = 256 << 20


def tq2_bytes(n, k):
    return n * (k // 128) * 34


KERNEL_SOURCES = {  # files whose content defines each timed kernel
    "gemv_mt_kernel": ["tq2_gemv.hip", "decode.h", "internal.h", "layout.h"],
    "mfma_gemm_kernel": ["mfma_gemm.h", "mfma_gemm.hip", "decode.h", "bitsign.h", "internal.h", "layout.h"],
}
PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 256 << 20   # plain device-to-device copy used to calibrate FETCH_SIZE / WRITE_SIZE


def source_sha(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "bit_weight_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, name):
    """HBM bytes per launch from a committed counter summary, if the kernel source is unchanged."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha(kernel) or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """W eager warmup steps, then K steps captured in one HIP graph; the graph is
    replayed once untimed and then REPS times, each replay bracketed by HIP events
    on the launch stream and by device synchronisations.  The per-step time is
    the median replay / K (the minimum is reported too).  The graph removes host
    launch cost from the timed region; a step is one or more library calls (each
    one or more kernel launches).  Warmup, capture and replays use one stream.
    The same K steps issued eagerly from Python are timed too, as context."""

    REPS = 11

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(steps):
                fn(i)
        with torch.cuda.stream(side):
            graph.replay()  # untimed first replay
        torch.cuda.synchronize()
        regions = []
        t0 = time.perf_counter()
        for _ in range(self.REPS):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(side):
                start.record(side)
                graph.replay()
                end.record(side)
            torch.cuda.synchronize()
            regions.append(start.elapsed_time(end))
        wall = time.perf_counter() - t0
        del graph
        # the same steps issued eagerly (host launch cost included), for context
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            e0.record(side)
            for i in range(steps):
                fn(i)
            e1.record(side)
        torch.cuda.synchronize()
        med = float(np.median(regions))
        return dict(region_ms=med, region_ms_all=[round(r, 4) for r in regions], step_ms=med / steps,
                    step_ms_min=min(regions) / steps, reps=self.REPS, host_wall_s=wall,
                    eager_step_ms=e0.elapsed_time(e1) / steps)


DECODE_LAYERS = 2 * MALL_BYTES // tq2_bytes(4096, 4096) + 1   # 121 weights: 539 MB per pass
MLP_LAYERS = 2 * MALL_BYTES // tq2_bytes(14336, 4096) + 1     # 35 weights: 546 MB per pass


def bench_decode(torch, bw, steps, warmup, path):
    """A step is one pass over DECODE_LAYERS uploaded copies of the decode weight, one
    tq2_gemm call each: every copy was last read a whole pass (> 2x the Infinity
    Cache) earlier, so each call streams its weight from HBM."""
    aos, x_np = wl.decode_inputs()
    n, k = wl.DECODE["N"], wl.DECODE["K"]
    nbytes = tq2_bytes(n, k)
    layers = DECODE_LAYERS
    log(f"[decode] uploading {layers} copies of the {nbytes} B weight")
    ws = [bw.tq2_upload(aos, n, k) for _ in range(layers)]
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((1, n), device="cuda")

    def step(i):
        for w in ws:
            bw.tq2_gemm_path(w, x, y, path)

    t = Timer(torch).run(step, steps, warmup)
    for w in ws:
        w.close()
    call_ms = t["step_ms"] / layers
    t.update(bytes_per_call=nbytes, calls_per_step=layers, call_ms=call_ms, call_ms_min=t["step_ms_min"] / layers,
             gbs_step=nbytes / (call_ms * 1e-3) / 1e9,
             gbs_eager=nbytes * layers / (t["eager_step_ms"] * 1e-3) / 1e9)
    return t


def bench_prefill(torch, bw, steps, warmup):
    aos, x_np = wl.prefill_inputs()
    m, n, k = wl.PREFILL["M"], wl.PREFILL["N"], wl.PREFILL["K"]
    w = bw.tq2_upload(aos, n, k)
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((m, n), device="cuda")
    t = Timer(torch).run(lambda i: bw.tq2_gemm_path(w, x, y, bw.TQ2_PATH_MFMA), steps, warmup)
    w.close()
    flop = 2.0 * m * n * k
    t.update(flop_per_call=flop, tflops_step=flop / (t["step_ms"] * 1e-3) / 1e12)
    return t


def bench_dit(torch, bw, steps, warmup, m, n, k):
    """The DiT benchmark shapes of "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs" on the MFMA
    path (LCG weights, scale 0.0625)."""
    aos, x_np = wl.dit_weight(n, k), wl.dit_x(m, k)
    w = bw.tq2_upload(aos, n, k)
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((m, n), device="cuda")
    t = Timer(torch).run(lambda i: bw.tq2_gemm_path(w, x, y, bw.TQ2_PATH_MFMA), steps, warmup)
    w.close()
    flop = 2.0 * m * n * k
    t.update(flop_per_call=flop, tflops_step=flop / (t["step_ms"] * 1e-3) / 1e12)
    return t


def bench_mlp(torch, bw, steps, warmup, m, path):
    """A step is one pass over MLP_LAYERS uploaded copies of the weight (cold, as for
    the decode)."""
    aos, x_np = wl.mlp_inputs(m)
    n, k = wl.MLP["N"], wl.MLP["K"]
    nbytes = tq2_bytes(n, k)
    layers = MLP_LAYERS
    ws = [bw.tq2_upload(aos, n, k) for _ in range(layers)]
    x = torch.from_numpy(x_np).cuda()
    y = torch.empty((m, n), device="cuda")

    def step(i):
        for w in ws:
            bw.tq2_gemm_path(w, x, y, path)

    t = Timer(torch).run(step, steps, warmup)
    for w in ws:
        w.close()
    call_ms = t["step_ms"] / layers
    t.update(bytes_per_call=nbytes, calls_per_step=layers, call_ms=call_ms, call_ms_min=t["step_ms_min"] / layers,
             gbs_step=nbytes / (call_ms * 1e-3) / 1e9, tflops_step=2.0 * m * n * k / (call_ms * 1e-3) / 1e12)
    return t


def bench_blr(torch, bw, steps, warmup):
    d = wl.blr_inputs()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bu, bv = dev(d["bits_u"].view(np.int32)), dev(d["bits_v"].view(np.int32))
    h, l, g, x = dev(d["h"]), dev(d["l"]), dev(d["g"]), dev(d["x"])
    m, d_in = d["x"].shape
    d_out, r = d["h"].size, d["l"].size
    y = torch.empty((m, d_out), device="cuda")
    t = Timer(torch).run(lambda i: bw.blr_forward(bu, bv, h, l, g, x, y), steps, warmup)
    flop = 2.0 * m * r * (d_in + d_out)
    t.update(flop_per_call=flop, tflops_step=flop / (t["step_ms"] * 1e-3) / 1e12)
    return t


def dense_baseline(torch, bw, steps, m, n, k, aos, x_np, reps=5):
    """The unfused alternative: decode the weight to dense f32 (tq2_dequant), cast it to
    f16, multiply with torch.matmul (the vendor GEMM, called as a library), cast y back to
    f32.  Timed eagerly (no graph capture of the library GEMM), median of `reps` runs of
    `steps` calls; the weight and activations are resident in HBM."""
    w = bw.tq2_upload(aos, n, k)
    x = torch.from_numpy(x_np).cuda()
    wf = torch.empty((n, k), dtype=torch.float32, device="cuda")
    w16 = torch.empty((n, k), dtype=torch.float16, device="cuda")
    x16 = torch.empty((m, k), dtype=torch.float16, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def step():
        bw.tq2_dequant(w, wf)
        w16.copy_(wf)
        x16.copy_(x)
        y.copy_(torch.matmul(x16, w16.t()))

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / steps)
    w.close()
    return float(np.median(times))


def context_floors(torch, steps=500):
    """What the box itself allows, measured the same way as the workloads: the
    per-launch cost of a one-element fill kernel in a replayed graph, and the
    HBM rates of a 1 GiB sum (read) and a 256 MiB copy (read + write)."""
    tiny = torch.zeros(1, device="cuda")
    t = Timer(torch).run(lambda i: tiny.fill_(float(i & 1)), steps, 10)
    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)

    def rate(fn, nbytes, reps=7):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return nbytes / (float(np.median(times)) * 1e-3) / 1e9

    read = rate(lambda: big.sum(), big.numel() * 4)
    copy = rate(lambda: b.copy_(a), 2 * CALIB_BYTES)
    del big, a, b
    return {"launch_floor_us": round(t["step_ms"] * 1e3, 3),
            "hbm_read_gbs": round(read, 1), "hbm_copy_gbs": round(copy, 1),
            "note": "launch floor: graph-replayed one-element fill; read: torch sum over 1 GiB f32; "
                    "copy: 256 MiB device copy, bytes read + written"}


def bench_blr_backward(torch, bw, steps, warmup):
    """Backward of the BLR workload (one path), dy ~ 1e-3 N(0, 1), gradient scale 1024."""
    d = wl.blr_inputs()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    m, d_in = d["x"].shape
    d_out, r = d["h"].size, d["l"].size
    bu, bv = dev(d["bits_u"].view(np.int32)[None]), dev(d["bits_v"].view(np.int32)[None])
    h, l, g, x = dev(d["h"][None]), dev(d["l"][None]), dev(d["g"][None]), dev(d["x"])
    dy = dev((np.random.default_rng(4).standard_normal((m, d_out)) * 1e-3).astype(np.float32))
    dh, dl, dg = (torch.zeros((1, n), device="cuda") for n in (d_out, r, d_in))
    dx = torch.empty((m, d_in), device="cuda")
    t = Timer(torch).run(lambda i: bw.blr_backward_paths(bu, bv, h, l, g, x, dy, dh, dl, dg, dx=dx), steps, warmup)
    flop = 2.0 * m * r * (d_in + d_out)  # the two gradient products; a and c are recomputed on top
    t.update(flop_per_call=flop, tflops_step=flop / (t["step_ms"] * 1e-3) / 1e12)
    return t


def bench_blr_saved(torch, bw, steps, warmup):
    """The layer forward that keeps a and c (blr_forward_paths_save) and the backward
    from them (blr_backward_paths_saved), one path, timed separately."""
    d = wl.blr_inputs()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    m, d_in = d["x"].shape
    d_out, r = d["h"].size, d["l"].size
    bu, bv = dev(d["bits_u"].view(np.int32)[None]), dev(d["bits_v"].view(np.int32)[None])
    h, l, g, x = dev(d["h"][None]), dev(d["l"][None]), dev(d["g"][None]), dev(d["x"])
    dy = dev((np.random.default_rng(4).standard_normal((m, d_out)) * 1e-3).astype(np.float32))
    y = torch.empty((m, d_out), device="cuda")
    saved = torch.empty(bw.blr_saved_size(1, m, d_in, d_out, r), dtype=torch.uint8, device="cuda")
    tf = Timer(torch).run(lambda i: bw.blr_forward_paths_save(bu, bv, h, l, g, x, y, saved), steps, warmup)
    dh, dl, dg = (torch.zeros((1, n), device="cuda") for n in (d_out, r, d_in))
    dx = torch.empty((m, d_in), device="cuda")
    tb = Timer(torch).run(lambda i: bw.blr_backward_paths_saved(bu, bv, h, l, g, x, dy, dh, dl, dg, saved, dx=dx),
                          steps, warmup)
    flop = 2.0 * m * r * (d_in + d_out)
    return {"forward_save_ms": tf["step_ms"], "forward_save_ms_min": tf["step_ms_min"],
            "backward_saved_ms": tb["step_ms"], "backward_saved_ms_min": tb["step_ms_min"],
            "backward_saved_tflops_algorithmic": flop / (tb["step_ms"] * 1e-3) / 1e12}


def calib_copy(torch, reps=5):
    """Untimed device copies of known size, for scaling the HBM byte counters."""
    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def summarize_stats(csv_path, command, trace_path=None):
    """Text summary of a rocprofv3 --stats kernel table (average duration per kernel), with
    each kernel's median duration from the kernel trace when one is given (the median is
    not moved by the few dispatches the profiler itself delays)."""
    import csv

    rows = list(csv.DictReader(open(csv_path)))
    med = {}
    if trace_path:
        durs = {}
        for r in csv.DictReader(open(trace_path)):
            durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        med = {k: float(np.median(v)) / 1e3 for k, v in durs.items()}
    print(f"# rocprofv3 kernel statistics")
    print(f"# command: {command}")
    print(f"# {'kernel':<90s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"
          + (f" {'median_us':>9s}" if med else ""))
    for r in rows:
        line = (f"  {r['Name'][:90]:<90s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.3f} "
                f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f}")
        if med:
            line += f" {med.get(r['Name'], float('nan')):9.3f}"
        print(line)


def summarize_pmc(fetch_csv, write_csv, kernel, command_fetch, command_write):
    """HBM traffic per launch of `kernel` from FETCH_SIZE / WRITE_SIZE runs, scaled by
    what the same counters read for the plain copy of CALIB_BYTES."""
    import csv

    def values(path, name_part, counter):
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter]

    def mean_kib(path, name_part, counter):
        vals = values(path, name_part, counter)
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    def copy_kib(path, counter):
        # the runtime's device copy kernel; the calibration copies are its largest dispatches
        vals = values(path, "copyBuffer", counter)
        if not vals:
            return None
        top = [v for v in vals if v >= 0.9 * max(vals)]
        return sum(top) / len(top)

    f_k, nf = mean_kib(fetch_csv, kernel, "FETCH_SIZE")
    w_k, nw = mean_kib(write_csv, kernel, "WRITE_SIZE")
    f_c = copy_kib(fetch_csv, "FETCH_SIZE")
    w_c = copy_kib(write_csv, "WRITE_SIZE")
    kib = CALIB_BYTES / 1024
    ff = kib / f_c if f_c else None
    fw = kib / w_c if w_c else None
    print("# HBM traffic per launch from rocprofv3 counters, scaled by a plain copy of known size")
    print(f"# fetch command: {command_fetch}")
    print(f"# write command: {command_write}")
    print(f"kernel: {kernel}")
    print(f"source_sha: {source_sha(kernel.split('<')[0])}")
    print(f"dispatches_fetch: {nf}")
    print(f"dispatches_write: {nw}")
    print(f"fetch_kib_per_dispatch_raw: {f_k}")
    print(f"write_kib_per_dispatch_raw: {w_k}")
    print(f"copy_fetch_kib_raw: {f_c}")
    print(f"copy_write_kib_raw: {w_c}")
    print(f"copy_bytes: {CALIB_BYTES}")
    print(f"fetch_scale: {ff}")
    print(f"write_scale: {fw}")
    if f_k is not None and w_k is not None and ff and fw:
        print(f"hbm_bytes_per_launch: {(f_k * ff + w_k * fw) * 1024:.0f}")


def summarize_counters(csv_paths, kernel, commands):
    """Per-dispatch averages of rocprofv3 --pmc counters for one kernel, from one or
    more counter passes, and the MFMA busy fraction: SQ_VALU_MFMA_BUSY_CYCLES (summed
    over the chip's 1024 SIMDs; it equals 32 cycles per 32x32x16 MFMA) over the
    GPU-active cycles of one XCD (GRBM_GUI_ACTIVE reads the sum over the 8 XCDs)."""
    import csv

    vals = {}
    for path in csv_paths.split(","):
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    print("# rocprofv3 counters per dispatch")
    for c in commands.split(";;"):
        print(f"# command: {c.strip()}")
    print(f"kernel: {kernel}")
    for name in sorted(vals):
        v = vals[name]
        print(f"{name}: {sum(v) / len(v):.6g}   (dispatches: {len(v)})")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        print(f"mfma_busy_fraction: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (avg['GRBM_GUI_ACTIVE'] / 8 * 1024):.4f}")
    if "SQ_INSTS_MFMA" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        print(f"mfma_busy_cycles_per_mfma_instruction: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.2f}")
    if "SQ_WAIT_INST_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
        print(f"wave_cycles_waiting_fraction: {avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.4f}")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, budget_s):
    """Calls of fn until budget_s has passed: (calls, seconds)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            return calls, dt


def cpu_baseline(budget_s=12.0):
    """The oracle, as it stands (never tuned), on bounded samples of the workloads:
    the decode on all cores (the headline unit) and on one thread, a row subset of
    the prefill and a few tokens of the BLR layer forward on all cores.  Same
    numerators as the GPU lines (packed weight bytes, algorithmic flop)."""
    import oracle

    cores = oracle.set_threads(os.cpu_count() or 1)
    aos, x = wl.decode_inputs()
    n, k = wl.DECODE["N"], wl.DECODE["K"]
    rows = 512                                   # first rows of the decode weight
    sub = aos[: tq2_bytes(rows, k)]
    calls, dt = _timed(lambda: oracle.gemm(sub, rows, k, x), budget_s * 0.4)
    gbs = calls * tq2_bytes(rows, k) / dt / 1e9
    oracle.set_threads(1)
    c1, dt1 = _timed(lambda: oracle.gemm(sub[: tq2_bytes(64, k)], 64, k, x), budget_s * 0.2)
    gbs1 = c1 * tq2_bytes(64, k) / dt1 / 1e9
    oracle.set_threads(cores)
    paos, px = wl.prefill_inputs()
    pm, prow = 8, 256                            # 8 of 2048 tokens x 256 of 4096 weight rows
    psub, pxs = paos[: tq2_bytes(prow, k)], px[:pm].copy()
    cp, dtp = _timed(lambda: oracle.gemm(psub, prow, k, pxs), budget_s * 0.2)
    pgf = cp * 2.0 * pm * prow * k / dtp / 1e9
    d = wl.blr_inputs()
    bm = 2                                       # 2 of 512 tokens
    bd = dict(d, x=d["x"][:bm].copy())
    cb, dtb = _timed(lambda: oracle.blr_forward(**bd), budget_s * 0.2)
    r, d_in, d_out = d["l"].size, d["x"].shape[1], d["h"].size
    bgf = cb * 2.0 * bm * r * (d_in + d_out) / dtb / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"M=1 decode, first {rows} of {n} weight rows (K={k}), {calls} calls in {dt:.1f} s on "
                      f"{cores} threads; f64 accumulation, OpenMP over outputs",
            "cpu_model": cpu_model(),
            "single_thread": {"value": gbs1, "unit": "GB/s",
                              "sample": f"M=1 decode, first 64 weight rows, {c1} calls in {dt1:.1f} s on 1 thread"},
            "prefill": {"value": pgf, "unit": "GFLOP/s",
                        "sample": f"M={pm} of 2048 tokens x {prow} of 4096 weight rows, K={k}, {cp} calls in "
                                  f"{dtp:.1f} s on {cores} threads"},
            "blr_forward": {"value": bgf, "unit": "GFLOP/s",
                            "sample": f"M={bm} of 512 tokens, d_in=d_out={d_in}, r={r}, {cb} calls in {dtb:.1f} s "
                                      f"on {cores} threads (algorithmic flop 2*M*r*(d_in+d_out))"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="decode,prefill,mlp,dit,blr,dense,cpu")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--summarize-stats", nargs="+", metavar="CSV COMMAND [TRACE_CSV]",
                    help="print a text summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "CMD_F", "CMD_W"),
                    help="print HBM traffic per launch from two counter runs and exit")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("CSVS", "KERNEL", "COMMANDS"),
                    help="print per-dispatch counter averages of KERNEL (CSVs comma-separated, commands ';;'-separated)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the ternary GEMM "
              f"shards along N with no exchange, so each GPU runs this same kernel on its N/G rows",
              file=sys.stderr)
        sys.exit(2)
    only = set(args.only.split(","))

    import torch

    import bit_weight_gemm_amd as bw

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")
    K, W = args.steps, args.warmup
    out = {}
    if "calib" in only:
        calib_copy(torch)
    if "decode" in only:
        out["decode_f32"] = bench_decode(torch, bw, K, W, bw.TQ2_PATH_F32)
        out["decode_mfma"] = bench_decode(torch, bw, max(K // 4, 2), max(W // 5, 1), bw.TQ2_PATH_MFMA)
        log(f"[decode] {json.dumps(out['decode_f32'])}")
    if "prefill" in only:
        out["prefill"] = bench_prefill(torch, bw, K, W)
        log(f"[prefill] {json.dumps(out['prefill'])}")
    if "mlp" in only:
        for m in wl.MLP["Ms"]:
            for name, path in (("f32", bw.TQ2_PATH_F32), ("mfma", bw.TQ2_PATH_MFMA)):
                out[f"mlp_m{m}_{name}"] = bench_mlp(torch, bw, max(K // 4, 2), max(W // 5, 1), m, path)
                log(f"[mlp M={m} {name}] {json.dumps(out[f'mlp_m{m}_{name}'])}")
    if "dit" in only:
        for (m, n, k) in wl.DIT_SHAPES:
            out[f"dit_{m}x{n}x{k}"] = bench_dit(torch, bw, max(K // 2, 5), 3, m, n, k)
            log(f"[dit {m}x{n}x{k}] {json.dumps(out[f'dit_{m}x{n}x{k}'])}")
    if "blr" in only:
        out["blr"] = bench_blr(torch, bw, max(K, 20), W)
        log(f"[blr] {json.dumps(out['blr'])}")
        out["blr_backward"] = bench_blr_backward(torch, bw, max(K, 20), W)
        log(f"[blr backward] {json.dumps(out['blr_backward'])}")
        out["blr_saved"] = bench_blr_saved(torch, bw, max(K, 20), W)
        log(f"[blr saved] {json.dumps(out['blr_saved'])}")

    line = {
        "metric": "TQ2 GEMM weight-GB/s (M=1) and TFLOP/s (M=2048), % of HBM/MFMA roofline",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64: codes iid over {-1,0,+1}, f16 scales U(0.01,0.1), x N(0,1))",
        "config": {"workload": f"decode GEMV: tq2_gemm M=1, N=4096, K=4096, TQ2_0_g128 weights (4,456,448 packed "
                               f"bytes per call); a step is one pass over {DECODE_LAYERS} separately uploaded "
                               f"weights, one call each (a {DECODE_LAYERS}-layer decode, 539 MB of weights)",
                   "path": "f32", "calls_per_step": DECODE_LAYERS},
    }
    if "decode_f32" in out:
        d = out["decode_f32"]
        line["value"] = round(d["gbs_step"], 2)
        line["ms_per_step"] = d["step_ms"]
        line["ms_per_step_min"] = d["step_ms_min"]
        line["us_per_call"] = round(d["call_ms"] * 1e3, 4)
        line["timing"] = (f"median (and min) over {d['reps']} replays of one HIP graph holding the K steps "
                          f"(K x {DECODE_LAYERS} calls), HIP events on the launch stream")
        line["roofline"] = {"bound": "hbm", "achieved": round(d["gbs_step"], 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(d["gbs_step"] / HBM_PEAK_GBS, 4),
                            "traffic": read_traffic("gemv_mt_kernel", "gemv_mt_decode_M1_traffic.txt"),
                            "kernel": "gemv_mt_kernel<2,1>", "launch_us": round(d["call_ms"] * 1e3, 4),
                            "launch_us_note": "average launch duration: HIP events around the replayed graph on "
                                              "its stream, divided by the launches it holds (back-to-back "
                                              "launches, gaps included)"}
        line["eager_value"] = round(d["gbs_eager"], 2)
    if "prefill" in out:
        p = out["prefill"]
        line["prefill"] = {"workload": "tq2_gemm M=2048, N=4096, K=4096 (MFMA f16 path, x staged to f16)",
                           "tflops": round(p["tflops_step"], 2), "ms_per_call": p["step_ms"],
                           "ms_per_call_min": p["step_ms_min"],
                           "roofline": {"bound": "mfma", "achieved": round(p["tflops_step"], 2),
                                        "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(p["tflops_step"] / MFMA_F16_PEAK_TFLOPS, 4),
                                        "kernel": "mfma_gemm_kernel<128,256>",
                                        "launch_us": round(p["step_ms"] * 1e3, 3)}}
    if "decode_mfma" in out:
        line["decode_mfma_path"] = {"gbs": round(out["decode_mfma"]["gbs_step"], 2),
                                    "us_per_call": round(out["decode_mfma"]["call_ms"] * 1e3, 3),
                                    "us_per_call_min": round(out["decode_mfma"]["call_ms_min"] * 1e3, 3)}
    for key in [k for k in out if k.startswith("mlp_")]:
        v = out[key]
        line[key] = {"gbs": round(v["gbs_step"], 2), "tflops": round(v["tflops_step"], 3),
                     "us_per_call": round(v["call_ms"] * 1e3, 3),
                     "us_per_call_min": round(v["call_ms_min"] * 1e3, 3),
                     "hbm_frac": round(v["gbs_step"] / HBM_PEAK_GBS, 4),
                     "cold": f"each step a pass over {MLP_LAYERS} uploaded copies"}
    for key in [k for k in out if k.startswith("dit_")]:
        v = out[key]
        line[key] = {"workload": f"tq2_gemm {key[4:]} (M x N x K, MFMA path, DiT benchmark shape)",
                     "tflops": round(v["tflops_step"], 2), "us_per_call": round(v["step_ms"] * 1e3, 2),
                     "us_per_call_min": round(v["step_ms_min"] * 1e3, 2),
                     "mfma_frac": round(v["tflops_step"] / MFMA_F16_PEAK_TFLOPS, 4)}
    if "blr" in out:
        b = out["blr"]
        line["blr"] = {"workload": "blr_forward M=512, d_in=d_out=4096, r=1024 (library-owned workspace)",
                       "tflops": round(b["tflops_step"], 2), "ms_per_call": b["step_ms"],
                       "ms_per_call_min": b["step_ms_min"],
                       "mfma_frac": round(b["tflops_step"] / MFMA_F16_PEAK_TFLOPS, 4)}
    if "decode" in only:
        line["context"] = context_floors(torch)
    if "dense" in only:
        try:
            aos, x_np = wl.decode_inputs()
            dec = dense_baseline(torch, bw, 200, 1, wl.DECODE["N"], wl.DECODE["K"], aos, x_np)
            aos, x_np = wl.prefill_inputs()
            pm, pn, pk = wl.PREFILL["M"], wl.PREFILL["N"], wl.PREFILL["K"]
            pre = dense_baseline(torch, bw, 20, pm, pn, pk, aos, x_np)
            line["dense_dequant_baseline"] = {
                "decode_us_per_call": round(dec * 1e3, 2), "prefill_us_per_call": round(pre * 1e3, 2),
                "prefill_tflops": round(2.0 * pm * pn * pk / (pre * 1e-3) / 1e12, 2),
                "what": "tq2_dequant to dense f32, cast to f16, torch.matmul f16 (vendor GEMM), y cast to "
                        "f32; eager, weight resident; the unfused alternative to tq2_gemm"}
        except Exception as e:  # a baseline only: report, do not fail the bench line
            line["dense_dequant_baseline"] = {"error": repr(e)[:200]}
    if "blr_backward" in out:
        b = out["blr_backward"]
        line["blr_backward"] = {"workload": "blr_backward_paths, one path, M=512, d_in=d_out=4096, r=1024 "
                                            "(a and c recomputed)",
                                "tflops_algorithmic": round(b["tflops_step"], 2),
                                "ms_per_call": b["step_ms"], "ms_per_call_min": b["step_ms_min"]}
    if "blr_saved" in out:
        b = out["blr_saved"]
        line["blr_saved"] = {"workload": "blr_forward_paths_save, then blr_backward_paths_saved from the kept a and c "
                                         "(one path, M=512, d_in=d_out=4096, r=1024)",
                             "forward_save_ms": b["forward_save_ms"], "forward_save_ms_min": b["forward_save_ms_min"],
                             "backward_saved_ms": b["backward_saved_ms"],
                             "backward_saved_ms_min": b["backward_saved_ms_min"],
                             "backward_saved_tflops_algorithmic": round(b["backward_saved_tflops_algorithmic"], 2)}
    if "cpu" in only:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
