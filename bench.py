#!/usr/bin/env python3
"""Benchmark of the W4A16 fused-QKV hot path on one MI355X.

A step is one kaio_qkv_w4a16 call on the prefill workload
(x f16[2048,4096], three packed-INT4 u32[512,4096] weights, three
f16[32,4096] scales, group 128 -> Q, K, V f16[2048,4096]); ``value`` is its
throughput in TFLOP/s (2*M*N*K*3 algorithmic flops per call).  The same JSON
line carries:

* ``roofline``     the prefill kernel against the dense f16 MFMA peak, with the
                   shader clock sampled while the kernel runs back to back and
                   the fraction against the peak at that clock, and against
                   MFMA work alone timed the same way (``mfma_alone``: the rate
                   the matrix cores sustain at the power limit);
* ``secondary``    the tiny 16x512x512 QKV (latency), decode (8 rows, weights
                   rotated over 21 sets so every call streams from HBM) next to
                   a plain streaming read of the same bytes, batched decode, the W8A16 sibling (decode and
                   prefill), the dense 4096^3 GEMM and its backward, and the
                   dequant backward (f32 and bf16, [16384, 8192], g=128) next to
                   a plain copy of the same bytes -- each against its own roof,
                   each with the CPU oracle timed on this host (``cpu_oracle``);
* ``cpu_baseline`` the float64 CPU oracle timed on this host's cores over the
                   prefill workload; the same leg compares the oracle's full
                   results with the GPU's (``parity`` entries: all outputs).

All inputs are seeded synthetic data already resident in device memory when
a timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 QKV TFLOP/s (prefill), weight GB/s (decode), % of MI355X roofline"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense f16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name: str) -> str:
    """Hash of a kernel source and common.hpp with comments and blank space removed, so that a
    comment edit does not void counters taken on the same code."""
    import re
    path = os.path.join(ROOT, "int4_group_quantized_w4a16_amd", "csrc", name)
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "int4_group_quantized_w4a16_amd", "csrc", "common.hpp")):
        with open(p, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


CONDITION_MS = 100.0


def condition(fn, ms=CONDITION_MS):
    """Runs fn() back to back, untimed, for about `ms` of GPU time.

    After an idle period (here: seconds of input generation on the host) the
    GPU needs ~10 ms of load to leave its low-power state: the first ~50
    prefill launches after idle take 210-280 us, the sustained rate is ~175 us
    (per-launch event series).  Every leg is therefore conditioned with its own
    work before its warm-up and timed steps, so that the timed steps measure
    the sustained rate of the kernel, not the power ramp."""
    import torch
    fn(0)                       # a first call may load code; it is not part of the estimate
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(3):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 3, 1e-3)
    for i in range(int(ms / per) + 1):
        fn(i)
    torch.cuda.synchronize()


def timed(fn, steps, warmup, stream, conditioned=False):
    """Average duration (ms) of fn() over `steps` back-to-back launches, HIP events on `stream`."""
    import torch
    if not conditioned:
        condition(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def timed_graph(fn, calls, replays, stream):
    """Average duration (ms) per fn() call when `calls` calls are captured in one HIP graph
    and the graph is replayed `replays` times (no host launch gaps between kernels)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    condition(lambda i: g.replay())
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (calls * replays)


def measured_traffic(kernel: str, src: str, algorithmic_bytes: float):
    """HBM bytes per launch from committed rocprofv3 PMC counters, or None if absent/stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash(src):
        return None
    return t.get("bytes_per_launch")


def host_cores():
    """Cores this process may run on (the oracle's BLAS and numpy use them)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def best_of(fn, runs):
    """Shortest wall time of `runs` calls of fn() (seconds) and the last result."""
    best, out = None, None
    for _ in range(runs):
        t0 = time.perf_counter()
        out = fn()
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return best, out


def oracle_entry(value, unit, seconds, sample):
    return {"value": round(value, 6), "unit": unit, "cores": host_cores(), "blas_threads": blas_threads(),
            "kind": "oracle", "seconds": round(seconds, 3), "sample": sample}


def cpu_baseline(inp, budget_s: float):
    """The float64 oracle on the prefill workload (all rows when they fit the budget), in TFLOP/s."""
    import numpy as np
    from oracle.qkv import qkv_project
    M, N, K = inp.shape
    probe = min(M, 128)
    t0 = time.perf_counter()
    qkv_project(inp.x, inp.w, inp.s, rows=np.arange(probe), with_abs=False)
    t_probe = time.perf_counter() - t0
    # the probe's time includes the fixed cost of dequantizing the weights, so
    # scaling it by rows over-estimates: a safe bound for the sample size
    rows = M if t_probe * M / probe <= budget_s else max(probe, int(M * budget_s / (t_probe * M / probe)))
    runs, spent = 0, 0.0
    while runs == 0 or (spent < budget_s and runs < 50):
        t0 = time.perf_counter()
        qkv_project(inp.x, inp.w, inp.s, rows=np.arange(rows), with_abs=False)
        spent += time.perf_counter() - t0
        runs += 1
    flops = 2.0 * rows * N * K * 3 * runs
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": host_cores(),
            "blas_threads": blas_threads(), "kind": "oracle",
            "sample": f"float64 oracle (numpy dequantize + f64 matmul, Y only), rows 0..{rows - 1} of the "
                      f"{M}-row prefill workload, {runs} run(s), {spent:.1f} s"}


def qkv_parity(outs, inp, bits=4):
    """All outputs against the oracle: violations, max |d|/tol, and the share equal to RNE_f16(Y*)."""
    import numpy as np
    from oracle import compare
    from oracle.qkv import qkv_project
    ys, ts = qkv_project(inp.x, inp.w, inp.s, bits=bits)
    bad, worst, equal, total = 0, 0.0, 0, 0
    for o, y, t in zip(outs, ys, ts):
        b, r = compare.excess(o, y, compare.qkv_tolerance(y, t))
        bad += b
        worst = max(worst, r)
        equal += int(compare.bits_equal(o, y.astype(np.float16)).sum())
        total += o.size
    return {"checked": total, "violations": bad, "max_ratio_to_tol": round(worst, 4),
            "bit_equal_to_rne_f16_of_oracle": round(equal / total, 6)}


def shader_clock_under(work, stream, dev, probes=6, probe_us=1000):
    """Shader clock while `work()` keeps the GPU busy: probe waves on a side stream (one
    wave each, no LDS, so they run beside the kernel's workgroups) count shader cycles
    against the real-time counter; returns their median in MHz, or None."""
    import ctypes
    import torch
    L = roof_lib()
    if L is None:
        return None
    khz = L.kaio_roof_wall_clock_khz()
    if khz <= 0:
        return None
    out = torch.zeros((probes, 4), dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    ticks = int(probe_us * khz / 1000)
    side.wait_stream(stream)
    work(0)                                   # queue the first part of the load
    with torch.cuda.stream(side):
        for i in range(probes):
            st = L.kaio_roof_clock_probe(ctypes.c_void_p(out[i].data_ptr()), ctypes.c_ulonglong(ticks),
                                         ctypes.c_void_p(side.cuda_stream))
            if st != 0:
                return None
    work(1)                                   # and the rest behind the probes
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    mhz = sorted(float(c) / float(r) * khz / 1000.0 for c, r, _, _ in v if r > 0)
    if not mhz:
        return None
    return {"median_mhz": round(mhz[len(mhz) // 2], 1), "min_mhz": round(mhz[0], 1), "max_mhz": round(mhz[-1], 1),
            "probes": len(mhz), "probe_us": probe_us,
            "source": "probe waves beside the back-to-back kernel: shader-clock counter (s_memtime) over the "
                      "real-time counter (s_memrealtime)"}


def roof_lib():
    import ctypes
    path = os.path.join(ROOT, "int4_group_quantized_w4a16_amd", "libkaio_roof.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.kaio_roof_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    L.kaio_roof_stream_read.restype = ctypes.c_int
    L.kaio_roof_sink_bytes.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.c_int]
    L.kaio_roof_sink_bytes.restype = ctypes.c_size_t
    L.kaio_roof_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
    L.kaio_roof_clock_probe.restype = ctypes.c_int
    L.kaio_roof_wall_clock_khz.argtypes = []
    L.kaio_roof_wall_clock_khz.restype = ctypes.c_int
    L.kaio_roof_strip_read.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_uint, ctypes.c_uint, ctypes.c_int,
                                                               ctypes.c_void_p, ctypes.c_void_p]
    L.kaio_roof_strip_read.restype = ctypes.c_int
    L.kaio_roof_strip_sink_bytes.argtypes = [ctypes.c_uint, ctypes.c_int]
    L.kaio_roof_strip_sink_bytes.restype = ctypes.c_size_t
    L.kaio_roof_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.kaio_roof_mfma.restype = ctypes.c_int
    L.kaio_roof_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.kaio_roof_mfma_flops.restype = ctypes.c_double
    return L


def mfma_roof(steps, stream, dev, iters=256, workgroups=2048):
    """MFMA work alone (dense f16 16x16x32 MFMAs on register operands, no memory traffic),
    conditioned and timed like the prefill, with the shader clock under it: the rate the matrix
    cores sustain under the chip's power limit when nothing else moves.  One launch (256
    iterations, 2048 workgroups of 4 waves) is ~275 GFLOP, about a prefill call's duration."""
    import ctypes
    import torch
    L = roof_lib()
    if L is None:
        return None
    sink = torch.empty((workgroups * 256,), dtype=torch.float32, device=dev)

    def fn(i):
        st = L.kaio_roof_mfma(sink.data_ptr(), iters, workgroups, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"kaio_roof_mfma failed ({st})")

    def sustained(part):
        for i in range(20 if part == 0 else 300):
            fn(i)
    fn(0)
    torch.cuda.synchronize()
    clk = shader_clock_under(sustained, stream, dev)
    condition(fn, 40.0)
    ms, _ = timed(fn, steps, 3, stream, conditioned=True)
    tf = L.kaio_roof_mfma_flops(iters, workgroups) / (ms * 1e-3) / 1e12
    log(f"[bench] MFMA alone: {ms * 1e3:.1f} us/call, {tf:.1f} TFLOP/s ({tf / PEAK_F16_TFLOPS:.1%} of peak)"
        + (f", shader clock {clk['median_mhz']:.0f} MHz" if clk else ""))
    r = {"what": "v_mfma_f32_16x16x32_f16 alone on register operands, 8 chains per wave, "
                 f"{workgroups} x 4 waves, {iters} x 8 MFMAs per wave (libkaio_roof.so)",
         "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4)}
    if clk:
        r["sclk_median_mhz"] = clk["median_mhz"]
    return r


def strip_roof(wsets, replays, stream, dev):
    """Read of the rotated packed-weight sets themselves by column strips, timed like decode:
    64-column strips of one array (the decode kernel's weight reads, 256-byte row segments) and
    16-column strips of all three (64-byte segments).  us per call and GB/s of the weights."""
    import ctypes
    import torch
    L = roof_lib()
    if L is None:
        return None
    rows, cols = wsets[0][0].shape
    nbytes = 3 * rows * cols * 4
    res = {"bytes": nbytes}
    for sc in (64, 16):
        sink = torch.empty((L.kaio_roof_strip_sink_bytes(cols, sc) // 4 + 1,), dtype=torch.int32, device=dev)

        def call(i, sc=sc, sink=sink):
            w = wsets[i % len(wsets)]
            st = L.kaio_roof_strip_read(w[0].data_ptr(), w[1].data_ptr(), w[2].data_ptr(), rows, cols, sc,
                                        sink.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(f"kaio_roof_strip_read failed ({st})")
        ms = timed_graph(call, 4 * len(wsets), replays, stream)
        res[f"strip{sc}"] = {"us_per_call": round(ms * 1e3, 3), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return res


# (loads per thread, threads); a negative count: the same shape with non-temporal loads
READ_SHAPES = ((1, 256), (2, 256), (4, 256), (8, 256), (8, 1024), (-1, 256), (-2, 256), (-4, 256), (-8, 256),
               (-8, 1024))


def read_roof(nbytes, sets, replays, stream, dev):
    """Best plain streaming read of `nbytes` (rotated over `sets` buffers, like the decode
    weights) over a few launch shapes, timed exactly like decode: us per call and GB/s."""
    import ctypes
    import torch
    L = roof_lib()
    if L is None:
        return None
    nb = (nbytes + 15) // 16 * 16
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nb // 4,), dtype=torch.int32, device=dev) for _ in range(sets)]
    best = None
    for u, th in READ_SHAPES:
        sink = torch.empty((L.kaio_roof_sink_bytes(nb, u, th) // 4 + 1,), dtype=torch.int32, device=dev)

        def call(i, u=u, th=th, sink=sink):
            st = L.kaio_roof_stream_read(bufs[i % sets].data_ptr(), nb, sink.data_ptr(), u, th,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(f"kaio_roof_stream_read failed ({st})")
        ms = timed_graph(call, 4 * sets, replays, stream)
        if best is None or ms < best[0]:
            best = (ms, u, th)
    del bufs
    ms, u, th = best
    return {"us_per_call": round(ms * 1e3, 3), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes": nbytes, "launch": f"{abs(u)} x 16-byte loads per thread{' (non-temporal)' if u < 0 else ''}, "
                                       f"{th} threads per workgroup",
            "shapes_tried": len(READ_SHAPES)}


def vendor_dense(m, n, k, out_f32, steps, stream, dev, clock=False):
    """The dense f16 product of the same shape through torch (the ROCm BLAS library), timed the same
    way: context for the fused kernels (a dense f16 weight matrix is 4x the packed INT4 bytes and
    needs no unpack).  With `clock`, also the shader clock under it, measured as for the prefill.
    Returns None when torch cannot run it."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn((m, k), generator=g, device=dev, dtype=torch.float16)
    b = torch.randn((k, n), generator=g, device=dev, dtype=torch.float16)
    fn = (lambda i: torch.mm(a, b, out_dtype=torch.float32)) if out_f32 else (lambda i: torch.mm(a, b))
    try:
        fn(0)
        torch.cuda.synchronize()
    except (RuntimeError, TypeError) as e:
        log(f"[bench] vendor dense {m}x{n}x{k} not timed: {str(e).splitlines()[0][:120]}")
        return None
    clk = None
    if clock:
        def sustained(part):
            for i in range(20 if part == 0 else 300):
                fn(i)
        clk = shader_clock_under(sustained, stream, dev)
    ms, _ = timed(fn, steps, 3, stream)
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    log(f"[bench] vendor dense f16 {m}x{n}x{k} ({'f32' if out_f32 else 'f16'} out): "
        f"{ms * 1e3:.1f} us/call, {tf:.1f} TFLOP/s"
        + (f", shader clock {clk['median_mhz']:.0f} MHz" if clk else ""))
    r = {"what": f"torch.mm f16[{m},{k}] x f16[{k},{n}] -> {'f32' if out_f32 else 'f16'} (dense weights)",
         "us_per_call": round(ms * 1e3, 2), "tflops": round(tf, 2)}
    if clk:
        r["sclk_median_mhz"] = clk["median_mhz"]
    return r


def summarize(dirs):
    """Per-kernel summary of rocprofv3 CSV output: kernel_stats.csv, kernel_trace.csv (dispatches
    grouped by kernel and grid, with the median duration) and counter_collection.csv."""
    import csv
    import collections
    import glob
    import statistics
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            groups = collections.defaultdict(list)
            for r in csv.DictReader(open(f)):
                wg = max(int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]), 1)
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // wg
                groups[(r["Kernel_Name"], grid, wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            print(f"## {f} (dispatches grouped by kernel and grid)")
            print("| kernel | grid | calls | avg us | min us | median us | max us |")
            print("|---|---|---|---|---|---|---|")
            for (name, grid, wg), us in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
                print(f"| {name.replace('(anonymous namespace)::', '')[:100]} | {grid} x {wg} | {len(us)} | {sum(us) / len(us):.2f} | {min(us):.2f} | "
                      f"{statistics.median(us):.2f} | {max(us):.2f} |")
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            print(f"## {f}")
            print("| kernel | calls | avg us | min us | max us | share |")
            print("|---|---|---|---|---|---|")
            for r in csv.DictReader(open(f)):
                print(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                      f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            agg = collections.defaultdict(lambda: collections.defaultdict(float))
            names = {}
            for r in csv.DictReader(open(f)):
                agg[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
            per_kernel = collections.defaultdict(list)
            for dsp, vals in agg.items():
                per_kernel[names[dsp]].append(vals)
            print(f"## {f}")
            for k, lst in per_kernel.items():
                keys = sorted(lst[0])
                avg = {c: sum(v[c] for v in lst) / len(lst) for c in keys}
                print(f"- {k[:90]} ({len(lst)} dispatches): " +
                      ", ".join(f"{c}={avg[c]:.6g}" for c in keys))


# the kernel instantiation each workload runs (the bench's own calls also launch others)
TRAFFIC_KERNELS = {"qkv_prefill": "qkv_prefill_kernel<4, 8,", "qkv_decode": "qkv_decode_kernel<4, 1, 1, 4, 16,"}


def write_traffic(key: str, src: str, fetch_dir: str, write_dir: str, command: str):
    """Record HBM bytes per launch of one kernel from two rocprofv3 --pmc runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one counter per run) are each
    scaled by what the same counter reads for the 256 MiB calibration copy of
    `--copy-calibration` in the same run; the entry is stamped with the kernel
    source hash so that bench.py stops using it once the kernel changes."""
    import csv
    import collections
    import glob

    def per_dispatch(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals, names = collections.defaultdict(float), {}
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
        kern = [v for dsp, v in vals.items() if TRAFFIC_KERNELS[key] in names[dsp]]
        copy = [v for dsp, v in vals.items() if "copy" in names[dsp].lower()]
        if not kern or not copy:
            raise SystemExit(f"{counter}: no {key} dispatch or no calibration copy under {d}")
        return sum(kern) / len(kern), max(copy), len(kern)

    calib_kib = (256 << 20) / 1024
    fk, fc, nf = per_dispatch(fetch_dir, "FETCH_SIZE")
    wk, wc, nw = per_dispatch(write_dir, "WRITE_SIZE")
    fs, ws = calib_kib / fc, calib_kib / wc
    entry = {"source_hash": kernel_source_hash(src), "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
             "bytes_per_launch": int(fk * fs * 1024 + wk * ws * 1024),
             "read_bytes_per_launch": int(fk * fs * 1024), "write_bytes_per_launch": int(wk * ws * 1024),
             "dispatches": [nf, nw], "command": command}
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[key] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps({key: entry}, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roof", action="store_true",
                    help="skip the plain-read and copy ceilings (for profiler runs)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "batched", "w8", "gemm", "bwd"], default="all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 CSV output directories instead of benchmarking")
    ap.add_argument("--write-traffic", nargs=4, metavar=("KERNEL", "SOURCE", "FETCH_DIR", "WRITE_DIR"),
                    help="record HBM bytes per launch of qkv_prefill|qkv_decode (source file name under csrc/) "
                         "from FETCH_SIZE and WRITE_SIZE counter runs into profiles/traffic.json")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.write_traffic:
        key, src, fdir, wdir = args.write_traffic
        write_traffic(key, src, fdir, wdir,
                      f"rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d <dir> -o run -- python3 bench.py "
                      f"--only {key.split('_')[1]} --steps 3 --warmup 1 --no-cpu-baseline --no-roof --copy-calibration")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path: the QKV projection would shard by output columns with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int4_group_quantized_w4a16_amd as kaio
    from int4_group_quantized_w4a16_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int32) if a.dtype == np.uint32 else a)).to(dev)
    result = {}
    secondary = {}
    host = {}          # GPU results kept for the CPU leg's full comparisons
    replays = max(5, args.steps // 10)

    # ---- prefill: the step --------------------------------------------------------------
    c = workloads.QKV_PREFILL
    M, N, K = c["M"], c["N"], c["K"]
    log(f"[bench] generating prefill inputs {M}x{N}x{K}")
    inp = workloads.qkv_inputs(M, N, K, c["seed"])
    x, w, s = t(inp.x), [t(a) for a in inp.w], [t(a) for a in inp.s]
    outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
    step = lambda i: kaio.kaio_qkv_w4a16(x, *w, *s, *outs)
    flops = 2.0 * M * N * K * 3
    # conditioning (see condition()) doubles as the clock measurement: probe waves count
    # shader cycles beside ~60 ms of back-to-back prefill launches
    for i in range(3):
        step(i)
    torch.cuda.synchronize()

    def sustained(part):
        for i in range(20 if part == 0 else 300):
            step(i)
    clock = shader_clock_under(sustained, stream, dev)
    condition(step, 40.0)
    ms, wall = timed(step, args.steps, args.warmup, stream, conditioned=True)
    tflops = flops / (ms * 1e-3) / 1e12
    algo_bytes = inp.x.nbytes + sum(a.nbytes for a in inp.w) + sum(a.nbytes for a in inp.s) + 3 * M * N * 2
    log(f"[bench] prefill: {ms * 1e3:.1f} us/call, {tflops:.1f} TFLOP/s ({tflops / PEAK_F16_TFLOPS:.1%} of peak)")
    host["prefill"] = [o.cpu().numpy() for o in outs]
    traffic = measured_traffic("qkv_prefill", "qkv_prefill.hip", algo_bytes)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_F16_TFLOPS, 4),
            "traffic": traffic, "algorithmic_flops": flops, "algorithmic_bytes": algo_bytes,
            "kernel": "qkv_prefill_kernel", "launch_us": round(ms * 1e3, 2)}
    if clock:
        peak_clk = PEAK_F16_TFLOPS * clock["median_mhz"] / 2400.0
        log(f"[bench] shader clock under sustained prefill: {clock['median_mhz']:.0f} MHz "
            f"(peak there {peak_clk:.0f} TFLOP/s)")
        roof.update({"sclk": clock, "peak_at_sclk": round(peak_clk, 1),
                     "frac_at_sclk": round(tflops / peak_clk, 4)})
    if not args.no_roof:
        # Q|K|V as one dense [K, 3N] f16 matrix through the vendor library
        roof["vendor_dense_f16"] = vendor_dense(M, 3 * N, K, False, args.steps, stream, dev, clock=True)
        mr = mfma_roof(args.steps, stream, dev)
        if mr:
            roof["mfma_alone"] = mr
            roof["frac_of_mfma_alone"] = round(tflops / mr["tflops"], 4)
    result.update({
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "W4A16 fused QKV prefill: x f16[2048,4096], 3x packed int4 u32[512,4096], "
                               "3x f16 scales [32,4096], group 128 -> Q,K,V f16[2048,4096]",
                   "M": M, "N": N, "K": K, "group_size": 128},
        "roofline": roof,
    })
    del x, w, s, outs

    # ---- tiny QKV (16 x 512 x 512): a latency figure, calls replayed from a HIP graph -----------
    if args.only in ("all", "decode"):
        c = workloads.QKV_TINY
        tin = workloads.qkv_inputs(c["M"], c["N"], c["K"], c["seed"])
        xt, wt, stt = t(tin.x), [t(a) for a in tin.w], [t(a) for a in tin.s]
        ot = [torch.empty((c["M"], c["N"]), dtype=torch.float16, device=dev) for _ in range(3)]
        tms = timed_graph(lambda i: kaio.kaio_qkv_w4a16(xt, *wt, *stt, *ot), 64, replays, stream)
        host["tiny"] = [o.cpu().numpy() for o in ot]
        pl = kaio.kaio_qkv_plan(c["M"], c["N"], c["K"])
        log(f"[bench] tiny QKV 16x512x512: {tms * 1e3:.2f} us/call")
        secondary["qkv_tiny"] = {
            "workload": "x f16[16,512], 3x packed int4 u32[64,512], 3x f16 scales [4,512] -> Q,K,V f16[16,512]",
            "us_per_call": round(tms * 1e3, 3), "bound": "latency",
            "tflops": round(2.0 * c["M"] * c["N"] * c["K"] * 3 / (tms * 1e-3) / 1e12, 3),
            "form": pl["kernel"], "timing": "64 calls per HIP graph replay"}
        del xt, wt, stt, ot

    # ---- decode, rotated weights, and the plain read of the same bytes ----------------
    if args.only in ("all", "decode", "batched"):
        c = workloads.QKV_DECODE
        M, N, K, R = c["M"], c["N"], c["K"], c["rotate"]
        log(f"[bench] generating {R} decode weight sets {M}x{N}x{K}")
        dinp = workloads.qkv_inputs(M, N, K, c["seed"])
        x = t(dinp.x)
        sets = [([t(a) for a in dinp.w], [t(a) for a in dinp.s])]
        for j in range(1, R):
            wj, sj = workloads.qkv_weight_set(N, K, c["seed"] + j)
            sets.append(([t(a) for a in wj], [t(a) for a in sj]))
        outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        dstep = lambda i: kaio.kaio_qkv_w4a16(x, *sets[i % R][0], *sets[i % R][1], *outs)
        # a ~10 us kernel: time it inside a HIP graph so host launch gaps are not counted
        dms = timed_graph(dstep, 4 * R, replays, stream)
        dbytes = dinp.x.nbytes + sum(a.nbytes for a in dinp.w) + sum(a.nbytes for a in dinp.s) + 3 * M * N * 2
        gbs = dbytes / (dms * 1e-3) / 1e9
        log(f"[bench] decode: {dms * 1e3:.2f} us/call, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
        dstep(0)
        torch.cuda.synchronize()
        host["decode"] = [o.cpu().numpy() for o in outs]
        rr = None if args.no_roof else read_roof(dbytes, R, replays, stream, dev)
        if rr:
            log(f"[bench] plain read of the same {dbytes} bytes: {rr['us_per_call']:.2f} us/call, {rr['gbs']:.0f} GB/s")
        sr = None if args.no_roof else strip_roof([st[0] for st in sets], replays, stream, dev)
        if sr:
            log(f"[bench] the weights read by 64-column strips: {sr['strip64']['us_per_call']:.2f} us/call; "
                f"by 16-column strips: {sr['strip16']['us_per_call']:.2f} us/call")
        secondary["qkv_decode"] = {
            "workload": "x f16[8,4096], 3x u32[512,4096], 3x f16[32,4096]; 21 rotated weight sets, "
                        "84 calls per HIP graph replay",
            "us_per_call": round(dms * 1e3, 3), "value": round(gbs, 1), "unit": "GB/s",
            "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": dbytes, "tflops": round(2.0 * M * N * K * 3 / (dms * 1e-3) / 1e12, 3),
            "traffic": measured_traffic("qkv_decode", "qkv_decode.hip", dbytes),
            "read_roof": rr, "frac_of_read_roof": round(rr["us_per_call"] / (dms * 1e3), 4) if rr else None,
            "strip_read_roof": sr}
        # batched decode and prefill chunks on the same rotated weights (split-K kernel up to
        # m = 64, then the tile kernel in the form kaio_qkv_plan reports)
        batched = []
        for bm in ((16, 32, 64, 96, 128, 256, 512, 768, 1024, 1536) if args.only != "decode" else ()):
            xb = t(np.random.default_rng(c["seed"] + 100 + bm).standard_normal((bm, K)).astype(np.float16))
            ob = [torch.empty((bm, N), dtype=torch.float16, device=dev) for _ in range(3)]
            bstep = lambda i: kaio.kaio_qkv_w4a16(xb, *sets[i % R][0], *sets[i % R][1], *ob)
            bms = timed_graph(bstep, 4 * R, replays, stream)
            bbytes = bm * K * 2 + sum(a.nbytes for a in dinp.w) + sum(a.nbytes for a in dinp.s) + 3 * bm * N * 2
            bgbs = bbytes / (bms * 1e-3) / 1e9
            btf = 2.0 * bm * N * K * 3 / (bms * 1e-3) / 1e12
            log(f"[bench] batched decode m={bm}: {bms * 1e3:.2f} us/call, {bgbs:.0f} GB/s, {btf:.1f} TFLOP/s")
            pl = kaio.kaio_qkv_plan(bm, N, K)
            batched.append({"m": bm, "us_per_call": round(bms * 1e3, 3), "gbs": round(bgbs, 1),
                            "tflops": round(btf, 2), "hbm_frac": round(bgbs / PEAK_HBM_GBS, 4),
                            "form": pl["kernel"] if pl["kernel"] == "split_k" else
                            f"tile {pl['waves']} waves x {pl['rows']} rows x {pl['sets']} set(s), "
                            f"{pl['outputs']} output(s) per workgroup"})
            del xb, ob
        if batched:
            secondary["qkv_batched_decode"] = {
                "workload": "x f16[m,4096] for m = 16 ... 1536; weights and rotation as qkv_decode",
                "points": batched, "bound": "hbm"}
        del sets, x, outs

    # ---- W8A16 sibling: decode (rotated) and prefill ----------------------------------
    if args.only in ("all", "w8"):
        c = workloads.QKV8_DECODE
        M, N, K, R = c["M"], c["N"], c["K"], c["rotate"]
        log(f"[bench] generating {R} W8A16 decode weight sets {M}x{N}x{K}")
        d8 = workloads.qkv8_inputs(M, N, K, c["seed"])
        x = t(d8.x)
        sets = [([t(a) for a in d8.w], [t(a) for a in d8.s])]
        for j in range(1, R):
            wj, sj = workloads.qkv8_weight_set(N, K, c["seed"] + j)
            sets.append(([t(a) for a in wj], [t(a) for a in sj]))
        outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        dstep = lambda i: kaio.kaio_qkv_w8a16(x, *sets[i % R][0], *sets[i % R][1], *outs)
        dms = timed_graph(dstep, 4 * R, replays, stream)
        dbytes = d8.x.nbytes + sum(a.nbytes for a in d8.w) + sum(a.nbytes for a in d8.s) + 3 * M * N * 2
        gbs = dbytes / (dms * 1e-3) / 1e9
        log(f"[bench] W8A16 decode: {dms * 1e3:.2f} us/call, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
        dstep(0)
        torch.cuda.synchronize()
        host["w8_decode"] = [o.cpu().numpy() for o in outs]
        rr = None if args.no_roof else read_roof(dbytes, R, replays, stream, dev)
        sr8 = None if args.no_roof else strip_roof([st[0] for st in sets], replays, stream, dev)
        if sr8:
            log(f"[bench] the INT8 weights read by 64-column strips: {sr8['strip64']['us_per_call']:.2f} us/call")
        secondary["qkv8_decode"] = {
            "workload": "W8A16: x f16[8,4096], 3x u32[1024,4096] (INT8), 3x f16[32,4096]; 11 rotated weight "
                        "sets, 44 calls per HIP graph replay",
            "us_per_call": round(dms * 1e3, 3), "value": round(gbs, 1), "unit": "GB/s", "bound": "hbm",
            "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": dbytes,
            "read_roof": rr, "frac_of_read_roof": round(rr["us_per_call"] / (dms * 1e3), 4) if rr else None,
            "strip_read_roof": sr8}
        del sets, x, outs
        c = workloads.QKV8_PREFILL
        M, N, K = c["M"], c["N"], c["K"]
        p8 = workloads.qkv8_inputs(M, N, K, c["seed"])
        x, w, s = t(p8.x), [t(a) for a in p8.w], [t(a) for a in p8.s]
        outs = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(3)]
        pms, _ = timed(lambda i: kaio.kaio_qkv_w8a16(x, *w, *s, *outs), args.steps, args.warmup, stream)
        ptf = 2.0 * M * N * K * 3 / (pms * 1e-3) / 1e12
        log(f"[bench] W8A16 prefill: {pms * 1e3:.1f} us/call, {ptf:.1f} TFLOP/s")
        host["w8_prefill"] = [o.cpu().numpy() for o in outs]
        secondary["qkv8_prefill"] = {
            "workload": "W8A16: x f16[2048,4096], 3x u32[1024,4096] (INT8), 3x f16[32,4096] -> Q,K,V f16[2048,4096]",
            "us_per_call": round(pms * 1e3, 2), "value": round(ptf, 2), "unit": "TFLOP/s", "bound": "mfma",
            "peak": PEAK_F16_TFLOPS, "frac": round(ptf / PEAK_F16_TFLOPS, 4)}
        del x, w, s, outs

    # ---- dense GEMM ------------------------------------------------------------------------
    if args.only in ("all", "gemm"):
        c = workloads.GEMM_4096
        M, N, K = c["M"], c["N"], c["K"]
        a, b = workloads.gemm_inputs(M, N, K, c["seed"])
        ad, bd = t(a), t(b)
        cd = torch.empty((M, N), dtype=torch.float32, device=dev)
        gms, _ = timed(lambda i: kaio.kaio_gemm_f16f32(ad, bd, cd), max(10, args.steps // 2), 3, stream)
        gtf = 2.0 * M * N * K / (gms * 1e-3) / 1e12
        log(f"[bench] gemm 4096^3: {gms * 1e3:.1f} us/call, {gtf:.1f} TFLOP/s")
        host["gemm"] = cd.cpu().numpy()
        secondary["gemm_f16f32"] = {"workload": "A f16[4096,4096] x B f16[4096,4096] -> C f32",
                                    "us_per_call": round(gms * 1e3, 2), "value": round(gtf, 2),
                                    "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_F16_TFLOPS,
                                    "frac": round(gtf / PEAK_F16_TFLOPS, 4)}
        mfma_alone = result["roofline"].get("mfma_alone")
        if mfma_alone:
            secondary["gemm_f16f32"]["frac_of_mfma_alone"] = round(gtf / mfma_alone["tflops"], 4)
        if not args.no_roof:
            secondary["gemm_f16f32"]["vendor"] = [
                vendor_dense(M, N, K, f32, max(10, args.steps // 2), stream, dev) for f32 in (True, False)]
        # backward of the same product: grad f32[M,N] -> grad_a f16[M,K], grad_b f16[K,N]
        g = np.random.default_rng(c["seed"] + 1).standard_normal((M, N)).astype(np.float32)
        gd = t(g)
        gad = torch.empty((M, K), dtype=torch.float16, device=dev)
        gbd = torch.empty((K, N), dtype=torch.float16, device=dev)
        wsd = torch.empty((kaio.lib().kaio_gemm_f16f32_bwd_workspace_size(M, N),), dtype=torch.uint8, device=dev)
        bms, _ = timed(lambda i: kaio.kaio_gemm_f16f32_bwd(ad, bd, gd, gad, gbd, wsd),
                       max(10, args.steps // 2), 3, stream)
        btf = 4.0 * M * N * K / (bms * 1e-3) / 1e12
        log(f"[bench] gemm bwd 4096^3: {bms * 1e3:.1f} us/call, {btf:.1f} TFLOP/s")
        host["gemm_bwd"] = (gad.cpu().numpy(), gbd.cpu().numpy(), g)
        host["gemm_ab"] = (a, b)
        secondary["gemm_f16f32_bwd"] = {
            "workload": "grad f32[4096,4096] -> grad_a = f16(grad) . B^T, grad_b = A^T . f16(grad), f16 outputs "
                        "(cast + two GEMM launches)",
            "us_per_call": round(bms * 1e3, 2), "value": round(btf, 2), "unit": "TFLOP/s", "bound": "mfma",
            "peak": PEAK_F16_TFLOPS, "frac": round(btf / PEAK_F16_TFLOPS, 4)}
        if mfma_alone:
            secondary["gemm_f16f32_bwd"]["frac_of_mfma_alone"] = round(btf / mfma_alone["tflops"], 4)
        del ad, bd, cd, gd, gad, gbd, wsd

    # ---- dequant backward, and a plain copy of the same bytes ---------------------------------
    if args.only in ("all", "bwd"):
        c = workloads.DEQUANT_BWD
        for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            dy, sc = workloads.dequant_bwd_inputs(c["outer"], c["axis"], c["group"], c["seed"], dt)
            if dt == "bf16":
                dyd = torch.from_numpy(dy.view(np.int16)).to(dev).view(torch.bfloat16)
                scd = torch.from_numpy(sc.view(np.int16)).to(dev).view(torch.bfloat16)
            else:
                dyd, scd = t(dy), t(sc)
            dqd = torch.empty_like(dyd)
            bms, _ = timed(lambda i: kaio.kaio_dequant_group_bwd(dyd, scd, c["group"], dqd),
                           max(10, args.steps // 2), 3, stream)
            nbytes = 2 * dy.nbytes + sc.nbytes
            gbs = nbytes / (bms * 1e-3) / 1e9
            log(f"[bench] dequant bwd {dt}: {bms * 1e3:.1f} us/call, {gbs:.0f} GB/s")
            host[f"bwd_{dt}"] = (dy, sc, dqd.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16"
                                 else dqd.cpu().numpy())
            cms = None
            if not args.no_roof:
                cpy = torch.empty_like(dyd)
                cms, _ = timed(lambda i: cpy.copy_(dyd), max(10, args.steps // 2), 3, stream)
                del cpy
            secondary[f"dequant_group_bwd_{dt}"] = {
                "workload": f"dy, dq {dt}[16384,8192], scale [16384,64], g=128",
                "us_per_call": round(bms * 1e3, 2), "value": round(gbs, 1), "unit": "GB/s", "bound": "hbm",
                "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nbytes,
                "copy_roof": None if cms is None else {
                    "us_per_call": round(cms * 1e3, 2), "gbs": round(2 * dy.nbytes / (cms * 1e-3) / 1e9, 1),
                    "what": "torch copy_ of dy into a buffer like dq (same bytes read and written, scales aside)"}}
            del dyd, scd, dqd

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    result["secondary"] = secondary
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
        cpu_leg(result, secondary, host, inp, workloads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def cpu_leg(result, secondary, host, inp, workloads):
    """The oracle on every workload the GPU ran: its time on this host next to each GPU
    figure, and a comparison of its full results with the GPU's."""
    import numpy as np
    from oracle import compare
    from oracle.dequant_bwd import dequant_bwd
    from oracle.gemm import gemm
    from oracle.gemm_bwd import gemm_bwd
    from oracle.qkv import qkv_project

    if "prefill" in host:
        result["roofline"]["parity"] = qkv_parity(host["prefill"], inp)
        log(f"[bench] prefill parity (all outputs): {result['roofline']['parity']}")
    # tiny QKV: the oracle on the full problem, and the GPU's outputs against it
    c = workloads.QKV_TINY
    tin = workloads.qkv_inputs(c["M"], c["N"], c["K"], c["seed"])
    sec, _ = best_of(lambda: qkv_project(tin.x, tin.w, tin.s, with_abs=False), 3)
    tiny_oracle = oracle_entry(2.0 * c["M"] * c["N"] * c["K"] * 3 / sec / 1e9, "GFLOP/s", sec,
                               "tiny QKV 16x512x512, full problem, best of 3")
    if "tiny" in host:
        secondary["qkv_tiny"]["cpu_oracle"] = tiny_oracle
        secondary["qkv_tiny"]["parity"] = qkv_parity(host["tiny"], tin)
    else:
        secondary["qkv_tiny_cpu_oracle"] = tiny_oracle
    if "decode" in host:
        c = workloads.QKV_DECODE
        dinp = workloads.qkv_inputs(c["M"], c["N"], c["K"], c["seed"])
        sec, _ = best_of(lambda: qkv_project(dinp.x, dinp.w, dinp.s, with_abs=False), 3)
        d = secondary["qkv_decode"]
        d["cpu_oracle"] = oracle_entry(d["algorithmic_bytes"] / sec / 1e9, "GB/s", sec,
                                       "decode 8x4096x4096 (weight set 0), full problem, best of 3")
        d["parity"] = qkv_parity(host["decode"], dinp)
    if "w8_decode" in host:
        c = workloads.QKV8_DECODE
        d8 = workloads.qkv8_inputs(c["M"], c["N"], c["K"], c["seed"])
        sec, _ = best_of(lambda: qkv_project(d8.x, d8.w, d8.s, with_abs=False, bits=8), 3)
        d = secondary["qkv8_decode"]
        d["cpu_oracle"] = oracle_entry(d["algorithmic_bytes"] / sec / 1e9, "GB/s", sec,
                                       "W8A16 decode 8x4096x4096 (weight set 0), full problem, best of 3")
        d["parity"] = qkv_parity(host["w8_decode"], d8, bits=8)
    if "w8_prefill" in host:
        c = workloads.QKV8_PREFILL
        p8 = workloads.qkv8_inputs(c["M"], c["N"], c["K"], c["seed"])
        sec, _ = best_of(lambda: qkv_project(p8.x, p8.w, p8.s, with_abs=False, bits=8), 1)
        d = secondary["qkv8_prefill"]
        d["cpu_oracle"] = oracle_entry(2.0 * c["M"] * c["N"] * c["K"] * 3 / sec / 1e12, "TFLOP/s", sec,
                                       "W8A16 prefill 2048x4096x4096, full problem (Y only), one run")
        d["parity"] = qkv_parity(host["w8_prefill"], p8, bits=8)
    if "gemm" in host:
        a, b = host["gemm_ab"]
        sec, (cref, tref) = best_of(lambda: gemm(a, b), 1)
        d = secondary["gemm_f16f32"]
        d["cpu_oracle"] = oracle_entry(2.0 * a.shape[0] * b.shape[1] * a.shape[1] / sec / 1e12, "TFLOP/s", sec,
                                       "GEMM 4096^3, full problem (C and sum |a*b|), one run")
        bad, worst = compare.excess(host["gemm"], cref, compare.gemm_tolerance(tref))
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(tref > 0, np.abs(host["gemm"].astype(np.float64) - cref) / tref, 0.0)
        d["parity"] = {"checked": int(cref.size), "violations": bad, "max_ratio_to_tol": round(worst, 5),
                       "max_abs_diff_over_T": float(rel.max())}
        del cref, tref, rel
        ga, gb, g = host["gemm_bwd"]
        sec, ((da, ta), (db, tb)) = best_of(lambda: gemm_bwd(a, b, g), 1)
        d = secondary["gemm_f16f32_bwd"]
        d["cpu_oracle"] = oracle_entry(4.0 * a.shape[0] * b.shape[1] * a.shape[1] / sec / 1e12, "TFLOP/s", sec,
                                       "GEMM backward 4096^3, full problem (both gradients and their T), one run")
        bads, worsts = 0, 0.0
        for got, y, tt in ((ga, da, ta), (gb, db, tb)):
            bb, ww = compare.excess(got, y, compare.f16_tolerance(y, tt))
            bads, worsts = bads + bb, max(worsts, ww)
        d["parity"] = {"checked": int(da.size + db.size), "violations": bads, "max_ratio_to_tol": round(worsts, 4)}
    for dt in ("f32", "bf16"):
        if f"bwd_{dt}" not in host:
            continue
        dy, sc, got = host[f"bwd_{dt}"]
        rows = 2048                      # a bounded sample of rows: the f64 oracle takes ~1 s per 2048
        sec, ref = best_of(lambda: dequant_bwd(dy[:rows], sc[:rows], 128, dt), 1)
        d = secondary[f"dequant_group_bwd_{dt}"]
        nbytes = 2 * dy[:rows].nbytes + sc[:rows].nbytes
        d["cpu_oracle"] = oracle_entry(nbytes / sec / 1e9, "GB/s", sec,
                                       f"rows 0..{rows - 1} of the 16384-row workload, one run")
        eq = compare.bits_equal(got[:rows], ref)
        d["parity"] = {"checked": int(eq.size), "bit_exact": bool(eq.all()),
                       "note": "the tests compare all 134.2 M elements; the bench re-checks the timed sample"}


if __name__ == "__main__":
    main()
