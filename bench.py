"""Benchmark of the row-exact few-row mat-vec on one MI355X.

A step is one pass of the hot path over the workload's m set: one
row_exact_mv call per m (Q8_0 4096 x 4096 at m = 1, 4, 8 by default), each on
the next of R copies of the weights so that the weights come from HBM rather
than the 256 MB Infinity Cache (R copies >= 1 GiB).  Inputs are resident in
HBM before timing.  The timed steps are replayed from a HIP graph captured on
the bench stream (launch overhead off the clock); the step time is the wall
time between two stream synchronisations around the replay.

Prints one JSON line.  ``value`` is effective weight GB/s over the whole job
(weight bytes of every call / wall time).  ``roofline`` is for the step's
dominant (longest) kernel, whose mean duration comes from HIP events around
back-to-back launches on the bench stream: the HBM roof (8 TB/s) with
``achieved`` = algorithmic bytes (weights + x + y) per second, and, as a
secondary figure, the kernel's algorithmic flops (2nmk per batch entry) per
second against the published FP32 vector peak (157.3 TFLOP/s; the kernels
issue unpacked FMAs, whose roof is half of it).  ``attainable_read`` is the
fastest plain read of the same weight bytes (include/row_exact_probe.h), the
practical ceiling for the weight stream at this size.  ``host_us_per_call``
is the host time of one eager C-ABI call.  ``cpu_baseline`` times the oracle
(float64 CPU reference) on a bounded sample of the same workload, split by
output rows over the host threads one GPU's share of the machine allows.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
# Published FP32 vector peak of MI355X (packed FP32: two FMAs per lane per clock).
FP32_PUBLISHED_TFLOPS = 157.3
# FP32 FMA issue rate of the vector ALUs without packed FP32, which these
# kernels do not use: 256 CUs x 64 lanes x 2 flops x 2.4 GHz.
VALU_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
# Host threads one GPU's share of the box may use (16 CPUs per GPU).
HOST_THREADS_PER_GPU = 16
METRIC = "effective weight GB/s and % of HBM peak, quantized GEMV at m=1/4/8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="q8_0_4096x4096")
    ap.add_argument("--cold-bytes", type=float, default=1.0, help="GiB of weight copies to rotate through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target duration of the oracle sample")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--sweep", default="", help="write per-(workload, m) kernel timings to this JSON file")
    ap.add_argument("--schedule-sweep", default="",
                    help="time the default schedule against pinned packings for the workloads named with "
                         "--sweep-workloads (default: the held-out shapes) and write the results to this JSON file")
    ap.add_argument("--sweep-workloads", default="", help="comma-separated workload names for --schedule-sweep")
    ap.add_argument("--split-sweep", default="",
                    help="write the skinny-output comparison (default schedule, its reduction split, against "
                         "the best single-wave-row packing) to this JSON file")
    ap.add_argument("--lane-sweep", default="",
                    help="write the lane-map comparison (default schedule, its lanes per row, against the best "
                         "packing on the other lane map) for the half-step workloads to this JSON file")
    ap.add_argument("--ab", default="",
                    help="another build of the library (python -m quantized_few_row_amd._build --out PATH -D ...): "
                         "time the default calls of both builds, interleaved, for the workloads named with "
                         "--sweep-workloads and write the results to --ab-out")
    ap.add_argument("--ab-out", default="ab.json", help="JSON file for --ab")
    ap.add_argument("--ab-ms", default="1,2,4,8", help="comma-separated input row counts for --ab")
    ap.add_argument("--profile-only", action="store_true",
                    help="launch the timed steps eagerly and exit (for rocprofv3 runs)")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only run a plain device copy of this many MiB, --steps times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write profiles/traffic.json from four rocprofv3 --pmc csv output folders: FETCH_SIZE and "
                         "WRITE_SIZE of a --profile-only run, then of a --copy-calibration run of the size given "
                         "with --copy-calibration (no GPU needed)")
    return ap.parse_args()


def _code_tokens(text):
    """C/C++ source without its comments, whitespace runs collapsed (string
    and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash():
    """Hash of the HIP sources' code (comments and whitespace left out);
    traffic counters are reported only for the code they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_few_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, m):
    """HBM bytes per launch of the (workload, m) kernel from the committed
    rocprofv3 --pmc summary, or None when it is missing or was taken on other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("launches", {}).get(f"{workload}:m{m}")
    if ent is None or ent.get("kernel_source_hash", rec.get("kernel_source_hash")) != kernel_source_hash():
        return None
    return ent.get("hbm_bytes")


def _counter_rows(folder, counter):
    """(kernel name, value) of every dispatch in the rocprofv3 csv files under folder."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"bench.py: no {counter} rows under {folder}")
    return rows


def copy_calibration_bytes(mib):
    """Bytes the --copy-calibration run copies per launch."""
    return int(mib * (1 << 20)) // 16 * 16


def write_traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_bytes, workload="q8_0_4096x4096"):
    """HBM bytes per launch of the mat-vec kernels from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the counter reads for a plain
    device copy of known size (``--copy-calibration``), into profiles/traffic.json."""
    import statistics

    import workloads as wl
    def cal_factor(folder, counter):
        rows = _counter_rows(folder, counter)
        copies = [v for name, v in rows if "copy" in name.lower()]
        if not copies:  # the kernel launched most often is the copy
            names = [name for name, _ in rows]
            top = max(set(names), key=names.count)
            copies = [v for name, v in rows if name == top]
        return statistics.median(copies)
    fetch_factor = cal_factor(cal_fetch_dir, "FETCH_SIZE") * 1024 / cal_bytes
    write_factor = cal_factor(cal_write_dir, "WRITE_SIZE") * 1024 / cal_bytes
    w = wl.get(workload)
    launches = {}
    per = {}
    for folder, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for name, v in _counter_rows(folder, counter):
            mt = re.search(r"mv_kernel<\s*(\d+)\s*,\s*(\d+)", name)
            if mt:
                per.setdefault((int(mt.group(2)), counter), []).append(v)
    import quantized_few_row_amd as qfr
    xrs, xbs, yrs, ybs = w.strides(8)
    s = qfr.Strides(xrs, xbs, yrs, ybs)
    for m in sorted({m for m, _ in per}):
        fk = statistics.mean(per[(m, "FETCH_SIZE")])
        wk = statistics.mean(per[(m, "WRITE_SIZE")])
        fb, wb = fk * 1024 / fetch_factor, wk * 1024 / write_factor
        _, xb, yb = qfr.row_exact_required_bytes(w.wtype, w.n, w.k, m, w.batch, s)
        launches[f"{workload}:m{m}"] = {
            "hbm_bytes": int(round(fb + wb)), "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
            "fetch_size_kib": fk, "write_size_kib": wk, "dispatches": len(per[(m, "FETCH_SIZE")]),
            "algorithmic_bytes": w.weight_bytes + xb + yb}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec.pop("kernel_source_hash", None)
    rec["copy_calibration"] = {"bytes": cal_bytes, "fetch_factor": fetch_factor, "write_factor": write_factor}
    h = kernel_source_hash()
    old = rec.get("launches", {})
    rec["launches"] = {key: e for key, e in old.items() if not key.startswith(workload + ":")}
    for key, e in launches.items():
        e["kernel_source_hash"] = h
        rec["launches"][key] = e
    rec["launches"] = dict(sorted(rec["launches"].items()))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"copy_calibration": rec["copy_calibration"], "launches": launches}, indent=1))


def main():
    args = parse()
    if args.write_traffic:
        if not args.copy_calibration:
            raise SystemExit("bench.py: --write-traffic needs --copy-calibration MIB (the size of the calibration copy)")
        write_traffic(*args.write_traffic, copy_calibration_bytes(args.copy_calibration), workload=args.workload)
        return
    if args.schedule_sweep:
        names = [v for v in args.sweep_workloads.split(",") if v] or None
        schedule_sweep(args.schedule_sweep, names)
        return
    if args.split_sweep:
        names = [v for v in args.sweep_workloads.split(",") if v] or None
        split_sweep(args.split_sweep, names)
        return
    if args.lane_sweep:
        names = [v for v in args.sweep_workloads.split(",") if v] or None
        lane_sweep(args.lane_sweep, names)
        return
    if args.ab:
        names = [v for v in args.sweep_workloads.split(",") if v] or None
        ab_compare(args.ab, args.ab_out, names, [int(v) for v in args.ab_ms.split(",") if v])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU; the mat-vec shards by weight rows with no "
              "reduction, and multi-GPU runs are not part of it (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = copy_calibration_bytes(args.copy_calibration)
        a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"bench.py: copied {nbytes} bytes {args.steps} times", flush=True)
        return
    w = wl.get(args.workload)
    t, n, k, batch = w.wtype, w.n, w.k, w.batch
    ms = list(w.ms) if args.workload != "q8_0_4096x4096" else [1, 4, 8]
    xrs, xbs, yrs, ybs = w.strides(8)
    strides = qfr.Strides(xrs, xbs, yrs, ybs)
    wbytes = w.weight_bytes

    W = w.make_weights()
    x = w.make_x(8)
    stored = w.stored_weight_bytes
    copies = max(2, int(np.ceil(args.cold_bytes * (1 << 30) / stored)))
    Wd = torch.empty((copies, stored), dtype=torch.uint8, device=dev)
    src = torch.from_numpy(W.ravel()).to(dev)
    for c in range(copies):
        Wd[c].copy_(src)
    del src
    xd = torch.from_numpy(x.ravel().copy()).to(dev)
    ybufs = {}
    for m in ms:
        _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, strides)
        ybufs[m] = torch.zeros(yb // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    lib = qfr.load_library()

    # Raw C-ABI calls (the binding's per-call Python checks are done once here).
    import ctypes
    sp = ctypes.byref(strides)
    hs = stream.cuda_stream
    wptrs = [Wd[c].data_ptr() for c in range(copies)]
    xp = xd.data_ptr()
    yptrs = {m: ybufs[m].data_ptr() for m in ms}
    idd = torch.from_numpy(w.make_ids()).to(dev) if w.experts else None
    if w.fused_norm:
        rd = torch.from_numpy(w.make_residual(8).ravel().copy()).to(dev)
        gd = torch.from_numpy(w.make_norm_weight()).to(dev)
        hd = torch.empty_like(rd)
    if w.fused_norm:  # checked path once
        qfr.row_exact_mv_add_rmsnorm(t, Wd[0], xd, rd, gd, 1e-5, hd, ybufs[ms[0]], n, k, ms[0], batch, strides,
                                     stream=hs)
    elif w.experts:
        qfr.row_exact_mv_gather(t, Wd[0], w.experts, idd, xd, ybufs[ms[0]], n, k, ms[0], batch, strides, stream=hs)
    else:
        qfr.row_exact_mv(t, Wd[0], xd, ybufs[ms[0]], n, k, ms[0], batch, strides, stream=hs)

    def launch(i, m):
        if w.fused_norm:
            rc = lib.row_exact_mv_add_rmsnorm(int(t), wptrs[i % copies], xp, rd.data_ptr(), gd.data_ptr(),
                                              ctypes.c_float(1e-5), hd.data_ptr(), yptrs[m], n, k, m, batch, sp, hs)
        elif w.experts:
            rc = lib.row_exact_mv_gather(int(t), wptrs[i % copies], w.experts, idd.data_ptr(), xp, yptrs[m], n, k, m,
                                         batch, sp, hs)
        else:
            rc = lib.row_exact_mv(int(t), wptrs[i % copies], xp, yptrs[m], n, k, m, batch, sp, hs)
        if rc:
            raise qfr.RowExactError(rc, qfr.row_exact_last_error())

    def steps(first, count):
        i = first
        for s in range(count):
            for m in ms:
                launch(i, m)
                i += 1
        return i

    with torch.cuda.stream(stream):
        i = steps(0, args.warmup)
    torch.cuda.synchronize()

    if args.profile_only:
        with torch.cuda.stream(stream):
            steps(i, args.steps)
        torch.cuda.synchronize()
        print(f"bench.py: profile-only run of {args.steps} steps of {args.workload} done", flush=True)
        return

    # Per-kernel durations: for each m, the timed number of launches back to
    # back on the bench stream (cycling the weight copies) between one pair of
    # HIP events, queued behind a bounded spin kernel so that the GPU never
    # waits for the host; the mean launch duration is the span over the count.
    kernel_us = {}
    for m in ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(2e8))
            e0.record(stream)
            for s_ in range(args.steps):
                launch(i + s_, m)
            e1.record(stream)
        torch.cuda.synchronize()
        kernel_us[m] = e0.elapsed_time(e1) * 1e3 / args.steps

    # Attainable read rate for this many bytes: a plain read of the same cold
    # weight copies (include/row_exact_probe.h), fastest launch shape.
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rbytes = wbytes // 16 * 16
    read_us = []
    for shape in range(qfr.row_exact_stream_read_shapes()):
        reps = max(2 * copies, 50)
        with torch.cuda.stream(stream):
            for r in range(copies):
                qfr.row_exact_stream_read(wptrs[r], rbytes, sink.data_ptr(), shape, stream=hs)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(2e8))
            e0.record(stream)
            for r in range(reps):
                qfr.row_exact_stream_read(wptrs[r % copies], rbytes, sink.data_ptr(), shape, stream=hs)
            e1.record(stream)
        torch.cuda.synchronize()
        read_us.append(e0.elapsed_time(e1) * 1e3 / reps)
    attainable = rbytes / (min(read_us) * 1e-6) / 1e9

    # Host time of one eager call: the C-ABI call (validation, schedule, launch)
    # timed from Python in a loop of ctypes calls, next to the same loop over
    # an entry point that does nothing (ctypes' own cost).  The launches queue
    # behind a spin kernel, so the GPU never back-pressures the host.
    # Each m gets a spin of its own and at most 200 queued launches, so the
    # launch queue never fills (a full queue blocks the host on the GPU).
    host_us = {}
    reps_h = 200
    t0 = time.perf_counter()
    for r in range(reps_h):
        lib.row_exact_launch_count()
    floor = (time.perf_counter() - t0) / reps_h * 1e6
    for m in ms:
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(2e8))
            t0 = time.perf_counter()
            for r in range(reps_h):
                launch(i + r, m)
            host_us[f"m{m}"] = round((time.perf_counter() - t0) / reps_h * 1e6, 3)
        torch.cuda.synchronize()
    host_us["ctypes_floor"] = round(floor, 3)

    # Whole-job timing: graph replay of the same K steps (or eager with --eager).
    y_eager = {m: ybufs[m].clone() for m in ms}
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            steps(i, args.steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        timing = "eager launches"
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            steps(i, args.steps)
        torch.cuda.synchronize()
        g.replay()  # untimed first replay
        torch.cuda.synchronize()
        for m in ms:  # the graph recomputes the same outputs bit for bit
            assert torch.equal(ybufs[m].view(torch.int32), y_eager[m].view(torch.int32)), "graph replay differs"
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        timing = "hip graph replay"

    calls = args.steps * len(ms)
    value = wbytes * calls / wall / 1e9
    dom = max(ms, key=lambda m: kernel_us[m])
    _, xb_dom, yb_dom = qfr.row_exact_required_bytes(t, n, k, dom, batch, strides)
    alg_bytes = wbytes + xb_dom + yb_dom
    flops = {mm: 2.0 * n * k * mm * batch for mm in ms}
    achieved = alg_bytes / (kernel_us[dom] * 1e-6) / 1e9
    tflops = flops[dom] / (kernel_us[dom] * 1e-6) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded SplitMix64 / Box-Muller blocks of the workload recipe)",
        "config": {
            "workload": args.workload, "weight_type": wl.TYPE_NAMES[t], "n": n, "k": k, "batch": batch,
            "m": ms, "weight_bytes": wbytes, "cold_weight_copies": copies, "timing": timing,
            "parallelism": "single GPU",
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "attainable_read": {"GBps": round(attainable, 1), "bytes": rbytes, "us": round(min(read_us), 3),
                            "hbm_frac": round(attainable / HBM_PEAK_GBS, 4)},
        "per_m": {str(m): {"kernel_us": round(kernel_us[m], 3),
                           "weight_GBps": round(wbytes / (kernel_us[m] * 1e-6) / 1e9, 1),
                           "hbm_frac": round(wbytes / (kernel_us[m] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "frac_of_attainable_read": round(min(read_us) / kernel_us[m], 4),
                           "fp32_TFLOPs": round(flops[m] / (kernel_us[m] * 1e-6) / 1e12, 2),
                           "fp32_frac_of_published": round(flops[m] / (kernel_us[m] * 1e-6) / 1e12
                                                           / FP32_PUBLISHED_TFLOPS, 4)}
                  for m in ms},
        "host_us_per_call": host_us,
        "kernel_source_hash": kernel_source_hash(),
        "roofline": {
            "kernel": f"mv_kernel<{wl.TYPE_NAMES[t]}, m={dom}>",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload, dom),
            "algorithmic_bytes_per_launch": alg_bytes, "mean_launch_us": round(kernel_us[dom], 3),
            "alu": {"achieved": round(tflops, 2), "peak": FP32_PUBLISHED_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / FP32_PUBLISHED_TFLOPS, 4),
                    "frac_of_unpacked_fma_peak": round(tflops / VALU_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": flops[dom],
                    "note": "published FP32 peak counts packed FMAs (two per lane per clock); these kernels "
                            "issue unpacked FMAs, whose roof is 78.6 TFLOP/s"},
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, W, x, ms, args.cpu_seconds)
    if args.sweep:
        out["sweep_file"] = args.sweep
        sweep(args.sweep, args.steps)
    print(json.dumps(out), flush=True)


def host_threads():
    """Threads for the CPU baseline: the CPUs this process may run on, at most
    one GPU's share of the box."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return max(1, min(avail, HOST_THREADS_PER_GPU)), avail


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, W, x, ms, seconds):
    """The oracle on whole output rows of the same workload, split by output
    rows over the host threads (each thread calls the unchanged oracle on its
    row range; the calls run outside the interpreter lock): the first S rows
    at every m of the step, S chosen from a short single-thread probe so the
    multi-thread sample takes about ``seconds``.  The same sample is then run
    on one thread, and both results are checked identical."""
    import threading

    import numpy as np

    import oracle
    t, n, k, batch = w.wtype, w.n, w.k, w.batch
    xrs, xbs, _, _ = w.strides(8)
    rb = oracle.row_bytes(t, k)
    threads, avail = host_threads()
    host = {"nproc": os.cpu_count(), "cpus_available": avail, "cpu_model": cpu_model()}
    if w.experts:  # gathered product: whole calls, one thread
        ids = w.make_ids()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < seconds:
            for m in ms:
                oracle.matvec_gather(t, W, w.experts, ids, x.ravel(), n, k, m, batch, xrs, xbs)
            reps += 1
        el = time.perf_counter() - t0
        return {"value": round(rb * n * batch * len(ms) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": f"{w.name}: {reps} whole step(s) at m={list(ms)}, float64 "
                                            f"dequantize-then-dot, single thread, {el:.1f} s",
                "seconds": round(el, 2), **host}
    probe = max(1, min(n, 16))
    t0 = time.perf_counter()
    for m in ms:
        oracle.matvec(t, W, x.ravel(), n, k, m, batch, xrs, xbs, rows=(0, probe))
    per_row = (time.perf_counter() - t0) / probe
    # rows for about `seconds` on all threads (assuming a near-linear speed-up)
    rows = int(max(threads, min(n, seconds * threads / max(per_row, 1e-9))))
    reps = max(1, int(seconds * threads / max(per_row * rows, 1e-9)))
    bounds = [(rows * i // threads, rows * (i + 1) // threads) for i in range(threads)]
    got = {m: [None] * threads for m in ms}

    def work(i):
        lo, hi = bounds[i]
        for _ in range(reps):
            for m in ms:
                got[m][i] = oracle.matvec(t, W, x.ravel(), n, k, m, batch, xrs, xbs, rows=(lo, hi))[0]

    pool = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    t0 = time.perf_counter()
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    el = time.perf_counter() - t0
    wbytes = rb * rows * batch * len(ms) * reps
    out = {"value": round(wbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{w.name}: first {rows} of {n} output rows x {batch} batch(es) at m={list(ms)}, "
                     f"{reps} pass(es), float64 dequantize-then-dot, split by output rows over {threads} "
                     f"host threads, {el:.1f} s",
           "seconds": round(el, 2), **host}
    # the same sample on one thread (one pass), checked identical
    t0 = time.perf_counter()
    same = True
    for m in ms:
        y1 = oracle.matvec(t, W, x.ravel(), n, k, m, batch, xrs, xbs, rows=(0, rows))[0]
        for i, (lo, hi) in enumerate(bounds):
            same &= bool(np.array_equal(got[m][i][..., lo:hi], y1[..., lo:hi]))
    el1 = time.perf_counter() - t0
    out["single_thread"] = {"value": round(rb * rows * batch * len(ms) / el1 / 1e9, 4), "unit": "GB/s",
                            "cores": 1, "seconds": round(el1, 2),
                            "identical_to_multi_thread": same}
    return out


def sweep(path, steps):
    """Mean kernel time of every (workload, m) with cold weights (one pair of
    HIP events around back-to-back launches queued behind a spin kernel), next
    to the attainable read time of the same bytes."""
    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl
    res = []
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for w in wl.WORKLOADS:
        t, n, k, batch = w.wtype, w.n, w.k, w.batch
        xrs, xbs, yrs, ybs = w.strides(8)
        s = qfr.Strides(xrs, xbs, yrs, ybs)
        W = w.make_weights()
        copies = max(2, int(np.ceil((1 << 30) / w.stored_weight_bytes)))
        Wd = torch.from_numpy(W.ravel()).cuda().repeat(copies).view(copies, -1)
        xd = torch.from_numpy(w.make_x(8).ravel().copy()).cuda()
        idd = torch.from_numpy(w.make_ids()).cuda() if w.experts else None
        if w.fused_norm:
            rd = torch.from_numpy(w.make_residual(8).ravel().copy()).cuda()
            gd = torch.from_numpy(w.make_norm_weight()).cuda()
            hd = torch.empty_like(rd)

        def mv(i, y, m):
            if w.experts:
                qfr.row_exact_mv_gather(t, Wd[i % copies], w.experts, idd, xd, y, n, k, m, batch, s)
            elif w.fused_norm:
                qfr.row_exact_mv_add_rmsnorm(t, Wd[i % copies], xd, rd, gd, 1e-5, hd, y, n, k, m, batch, s)
            else:
                qfr.row_exact_mv(t, Wd[i % copies], xd, y, n, k, m, batch, s)

        rbytes = w.weight_bytes // 16 * 16
        reps = min(steps, 200)

        def span_us(fn):
            """Mean duration of reps back-to-back launches of fn(i)."""
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(2e8))
            a.record()
            for i in range(reps):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / reps

        read_us = []
        for shape in range(qfr.row_exact_stream_read_shapes()):
            for i in range(min(copies, 64)):
                qfr.row_exact_stream_read(Wd[i], rbytes, sink, shape)
            read_us.append(span_us(lambda i: qfr.row_exact_stream_read(Wd[i % copies], rbytes, sink, shape)))
        for m in sorted(set(w.ms) | {1, 4, 8}):
            _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, s)
            y = torch.zeros(yb // 4, dtype=torch.float32, device="cuda")
            for i in range(10):
                mv(i, y, m)
            us = span_us(lambda i: mv(i, y, m))
            sch = qfr.row_exact_schedule(t, n, k, m, batch)
            fl = 2.0 * n * k * m * batch
            res.append({"workload": w.name, "m": m, "kernel_us": round(us, 3),
                        "weight_GBps": round(w.weight_bytes / us / 1e3, 1),
                        "hbm_frac": round(w.weight_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                        "attainable_read_us": round(min(read_us), 3),
                        "frac_of_attainable_read": round(min(read_us) / us, 4),
                        "fp32_frac_of_published": round(fl / (us * 1e-6) / 1e12 / FP32_PUBLISHED_TFLOPS, 4),
                        "schedule": sch.asdict()})
            if w.fused_norm:
                # the same call as two launches on a work buffer, and the plain
                # product on x alone (what the normalisation costs)
                work = torch.empty(qfr.norm_work_bytes(k, m, batch), dtype=torch.uint8, device="cuda")
                us2 = span_us(lambda i: qfr.row_exact_mv_add_rmsnorm_ws(t, Wd[i % copies], xd, rd, gd, 1e-5, hd, y, n,
                                                                       k, m, batch, s, work=work))
                us0 = span_us(lambda i: qfr.row_exact_mv(t, Wd[i % copies], xd, y, n, k, m, batch, s))
                # the residual form (h := r, layer output x, w = w2 := g), same work buffer
                us3 = span_us(lambda i: qfr.row_exact_mv_residual_rmsnorm_ws(
                    t, Wd[i % copies], rd, xd, gd, None, gd, 1e-5, 1e-5, hd, y, n, k, m, batch, s, work=work))
                res[-1].update({"one_kernel_us": round(us, 3), "two_launch_us": round(us2, 3),
                                "plain_product_us": round(us0, 3), "residual_two_launch_us": round(us3, 3)})
            print(json.dumps(res[-1]), file=sys.stderr, flush=True)
        del Wd
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(res, f, indent=1)


def schedule_sweep(path, names=None):
    """The chooser against pinned packings.  For every m of each workload:
    the default schedule and pinned ones (rows per wave 1/2/4, 2/4/8 waves per
    workgroup, 1..32 workgroups per CU or one row group per wave, one or two
    LDS passes), each timed as the mean of back-to-back launches on cold
    weights (checked bitwise equal to the default: packing is inert); then
    the default and the three fastest pinned schedules again, in five
    interleaved rounds, median per schedule."""
    import ctypes
    import itertools
    import statistics

    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl
    names = names or list(wl.HELD_OUT)
    lib = qfr.load_library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.Stream()
    hs = stream.cuda_stream
    step = {wl.F16: 512, wl.Q8_0: 2048, wl.Q4_K: 4096, wl.Q6_K: 4096, wl.Q5_0: 2048, wl.F32: 256, wl.BF16: 512}
    res = []
    for name in names:
        w = wl.get(name)
        t, n, k, batch = w.wtype, w.n, w.k, w.batch
        xrs, xbs, yrs, ybs = w.strides(8)
        st = qfr.Strides(xrs, xbs, yrs, ybs)
        W = w.make_weights()
        copies = max(2, int(np.ceil((1 << 30) / w.stored_weight_bytes)))
        Wd = torch.from_numpy(W.ravel()).cuda().repeat(copies).view(copies, -1)
        wp = [Wd[c].data_ptr() for c in range(copies)]
        xd = torch.from_numpy(w.make_x(8).ravel().copy()).cuda()
        for m in w.ms:
            _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, st)
            y = torch.zeros(yb // 4, dtype=torch.float32, device="cuda")
            d = qfr.row_exact_schedule(t, n, k, m, batch)
            cands = {}
            # one pass, the default's pass length, half of it and one wave step
            kcs = {k, d.k_chunk, max(step[t], d.k_chunk // 2 // step[t] * step[t]), step[t]}
            for nr, wv, f in itertools.product((1, 2, 4), (2, 4, 8), (1, 2, 4, 8, 16, 32, 0)):
                for kc in sorted(kcs):
                    if kc < k and kc % step[t]:
                        continue
                    wgs = max(1, cus * f // wv // batch) if f else 1 << 30
                    s = qfr.Schedule(d.k_split, nr, wv, wgs, kc)
                    cands[(nr, wv, f, kc)] = s

            def run(s, i):
                if s is None:
                    return lib.row_exact_mv(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                            ctypes.byref(st), hs)
                return lib.row_exact_mv_scheduled(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                                  ctypes.byref(st), ctypes.byref(s), hs)

            def mean_us(s, reps=100):
                with torch.cuda.stream(stream):
                    for i in range(3):
                        run(s, i)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda._sleep(int(2e6))
                    e0.record(stream)
                    for i in range(reps):
                        run(s, i)
                    e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / reps

            with torch.cuda.stream(stream):
                run(None, 0)
            torch.cuda.synchronize()
            ref = y.clone()
            timed = {}
            for key, s in cands.items():
                with torch.cuda.stream(stream):
                    rc = run(s, 0)
                if rc:  # over the device's limits (refused before launch)
                    continue
                torch.cuda.synchronize()
                if not torch.equal(ref.view(torch.int32), y.view(torch.int32)):
                    raise SystemExit(f"bench.py: schedule {s} changed the bits of {name} m={m}")
                timed[key] = mean_us(s)
            best = sorted(timed, key=timed.get)[:3]
            rounds = {None: [], **{b: [] for b in best}}
            for _ in range(5):
                for key in rounds:
                    rounds[key].append(mean_us(cands[key] if key else None))
            med = {key: statistics.median(v) for key, v in rounds.items()}
            best_key = min(best, key=med.get)
            rec = {"workload": name, "m": m, "default": d.asdict(), "default_us": round(med[None], 3),
                   "best_pinned": cands[best_key].asdict(), "best_pinned_us": round(med[best_key], 3),
                   "default_over_best": round(med[None] / med[best_key], 4),
                   "candidates_timed": len(timed)}
            res.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
        del Wd
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(res, f, indent=1)


def split_sweep(path, names=None):
    """Skinny outputs: for every m of each workload, the default schedule
    (whose reduction split is derived from (type, k, n)) against pinned
    packings with the split at 1 (one wave per row; the bits then differ,
    within the tolerance) and with the derived split: rows per wave 1 / 2,
    1 / 2 / 4 / 8 waves per workgroup (multiples of the split), one round of
    workgroups, the default's LDS pass.  Each timed as the mean of
    back-to-back launches on cold weights; then the default and the best of
    each split again, in five interleaved rounds, median per schedule."""
    import ctypes
    import statistics

    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl
    names = names or list(wl.SKINNY)
    lib = qfr.load_library()
    stream = torch.cuda.Stream()
    hs = stream.cuda_stream
    res = []
    for name in names:
        w = wl.get(name)
        t, n, k, batch = w.wtype, w.n, w.k, w.batch
        xrs, xbs, yrs, ybs = w.strides(8)
        st = qfr.Strides(xrs, xbs, yrs, ybs)
        W = w.make_weights()
        copies = max(2, int(np.ceil((1 << 30) / w.stored_weight_bytes)))
        Wd = torch.from_numpy(W.ravel()).cuda().repeat(copies).view(copies, -1)
        wp = [Wd[c].data_ptr() for c in range(copies)]
        xd = torch.from_numpy(w.make_x(8).ravel().copy()).cuda()
        for m in w.ms:
            _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, st)
            y = torch.zeros(yb // 4, dtype=torch.float32, device="cuda")
            d = qfr.row_exact_schedule(t, n, k, m, batch)
            cands = {}
            for K in sorted({1, d.k_split}):
                for nr in (1, 2):
                    for wv in (1, 2, 4, 8):
                        if wv % K:
                            continue
                        wgs = max(1, -(-n // (nr * wv // K)))
                        cands[(K, nr, wv)] = qfr.Schedule(K, nr, wv, wgs, d.k_chunk)

            def run(s, i):
                if s is None:
                    return lib.row_exact_mv(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                            ctypes.byref(st), hs)
                return lib.row_exact_mv_scheduled(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                                  ctypes.byref(st), ctypes.byref(s), hs)

            def mean_us(s, reps=100):
                with torch.cuda.stream(stream):
                    for i in range(3):
                        run(s, i)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda._sleep(int(2e6))
                    e0.record(stream)
                    for i in range(reps):
                        run(s, i)
                    e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / reps

            timed = {}
            for key, s in cands.items():
                with torch.cuda.stream(stream):
                    rc = run(s, 0)
                torch.cuda.synchronize()
                if rc:  # over the device's limits (refused before launch)
                    continue
                timed[key] = mean_us(s)
            best = {K: min((key for key in timed if key[0] == K), key=timed.get) for K in {key[0] for key in timed}}
            rounds = {None: [], **{b: [] for b in best.values()}}
            for _ in range(5):
                for key in rounds:
                    rounds[key].append(mean_us(cands[key] if key else None))
            med = {key: statistics.median(v) for key, v in rounds.items()}
            rec = {"workload": name, "m": m, "default": d.asdict(), "default_us": round(med[None], 3),
                   "best_unsplit": cands[best[1]].asdict(), "best_unsplit_us": round(med[best[1]], 3),
                   "best_derived_split": cands[best[d.k_split]].asdict(),
                   "best_derived_split_us": round(med[best[d.k_split]], 3),
                   "unsplit_over_default": round(med[best[1]] / med[None], 4),
                   "candidates_timed": len(timed)}
            res.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
        del Wd
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(res, f, indent=1)


def lane_sweep(path, names=None):
    """Rows whose last 64-lane wave step is at most half full: for every m of
    each workload, the default schedule (lanes per row derived from the
    weight type, k and the split) against pinned packings on the other lane
    map (64 lanes per row where the default takes 32, 32 where it keeps 64;
    the bits then differ, within the tolerance) and on the derived one: rows
    per wave 1 / 2 / 4, 4 / 8 waves per workgroup, half, once and twice the
    default's workgroups per batch entry or one row group per wave, the
    default's LDS pass.  Each
    timed as the mean of back-to-back launches on cold weights; then the
    default and the best of each map again, in five interleaved rounds,
    median per schedule."""
    import ctypes
    import statistics

    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl
    names = names or list(wl.LANE_MAP)
    lib = qfr.load_library()
    stream = torch.cuda.Stream()
    hs = stream.cuda_stream
    res = []
    for name in names:
        w = wl.get(name)
        t, n, k, batch = w.wtype, w.n, w.k, w.batch
        xrs, xbs, yrs, ybs = w.strides(8)
        st = qfr.Strides(xrs, xbs, yrs, ybs)
        W = w.make_weights()
        copies = max(2, int(np.ceil((1 << 30) / w.stored_weight_bytes)))
        Wd = torch.from_numpy(W.ravel()).cuda().repeat(copies).view(copies, -1)
        wp = [Wd[c].data_ptr() for c in range(copies)]
        xd = torch.from_numpy(w.make_x(8).ravel().copy()).cuda()
        for m in sorted(set(w.ms) | {1, 2, 4, 8}):
            _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, st)
            y = torch.zeros(yb // 4, dtype=torch.float32, device="cuda")
            d = qfr.row_exact_schedule(t, n, k, m, batch)
            other = 32 if d.lanes_per_row == 64 else 64
            cands = {}
            wgs_set = sorted({max(1, d.workgroups_per_batch // 2), d.workgroups_per_batch,
                              2 * d.workgroups_per_batch, 1 << 30})
            for L in (d.lanes_per_row, other):
                for nr in (1, 2, 4):
                    for wv in (4, 8):
                        for wgs in wgs_set:
                            cands[(L, nr, wv, wgs)] = qfr.Schedule(d.k_split, nr, wv, wgs, d.k_chunk, L)

            def run(s, i):
                if s is None:
                    return lib.row_exact_mv(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                            ctypes.byref(st), hs)
                return lib.row_exact_mv_scheduled(t, wp[i % copies], xd.data_ptr(), y.data_ptr(), n, k, m, batch,
                                                  ctypes.byref(st), ctypes.byref(s), hs)

            def mean_us(s, reps=100):
                with torch.cuda.stream(stream):
                    for i in range(3):
                        run(s, i)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda._sleep(int(2e6))
                    e0.record(stream)
                    for i in range(reps):
                        run(s, i)
                    e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / reps

            timed = {}
            for key, s in cands.items():
                with torch.cuda.stream(stream):
                    rc = run(s, 0)
                torch.cuda.synchronize()
                if rc:  # over the device's limits (refused before launch)
                    continue
                timed[key] = mean_us(s)
            best = {L: min((key for key in timed if key[0] == L), key=timed.get) for L in {key[0] for key in timed}}
            rounds = {None: [], **{b: [] for b in best.values()}}
            for _ in range(5):
                for key in rounds:
                    rounds[key].append(mean_us(cands[key] if key else None))
            med = {key: statistics.median(v) for key, v in rounds.items()}
            bo, bd = best[other], best[d.lanes_per_row]
            rec = {"workload": name, "m": m, "default": d.asdict(), "default_us": round(med[None], 3),
                   "best_other_lanes": cands[bo].asdict(), "best_other_lanes_us": round(med[bo], 3),
                   "best_derived_lanes": cands[bd].asdict(), "best_derived_lanes_us": round(med[bd], 3),
                   "other_over_default": round(med[bo] / med[None], 4), "candidates_timed": len(timed)}
            res.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
        del Wd
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(res, f, indent=1)


def ab_compare(other_path, path, names=None, ms=(1, 2, 4, 8)):
    """The same default calls through this package's library (A) and another
    build of it (B, e.g. one with a code-generation switch overridden): for
    every workload and m, both outputs compared bit for bit, then five
    interleaved rounds of back-to-back launches on cold weights per build,
    median per build."""
    import ctypes
    import statistics

    import numpy as np
    import torch

    import quantized_few_row_amd as qfr
    import workloads as wl
    names = names or list(wl.LANE_MAP)
    libs = {"a": qfr.load_library(), "b": qfr.load_variant(other_path)}
    stream = torch.cuda.Stream()
    hs = stream.cuda_stream
    res = []
    for name in names:
        w = wl.get(name)
        t, n, k, batch = w.wtype, w.n, w.k, w.batch
        xrs, xbs, yrs, ybs = w.strides(8)
        st = qfr.Strides(xrs, xbs, yrs, ybs)
        W = w.make_weights()
        copies = max(2, int(np.ceil((1 << 30) / w.stored_weight_bytes)))
        Wd = torch.from_numpy(W.ravel()).cuda().repeat(copies).view(copies, -1)
        wp = [Wd[c].data_ptr() for c in range(copies)]
        xd = torch.from_numpy(w.make_x(8).ravel().copy()).cuda()
        idd = torch.from_numpy(w.make_ids()).cuda() if w.experts else None
        if w.fused_norm:
            rd = torch.from_numpy(w.make_residual(8).ravel().copy()).cuda()
            gd = torch.from_numpy(w.make_norm_weight()).cuda()
            hd = torch.empty_like(rd)
        for m in ms:
            _, _, yb = qfr.row_exact_required_bytes(t, n, k, m, batch, st)
            ys = {tag: torch.zeros(yb // 4, dtype=torch.float32, device="cuda") for tag in libs}

            def run(tag, i):
                lib, y = libs[tag], ys[tag].data_ptr()
                if w.experts:
                    return lib.row_exact_mv_gather(t, wp[i % copies], w.experts, idd.data_ptr(), xd.data_ptr(), y,
                                                   n, k, m, batch, ctypes.byref(st), hs)
                if w.fused_norm:
                    return lib.row_exact_mv_add_rmsnorm(t, wp[i % copies], xd.data_ptr(), rd.data_ptr(),
                                                        gd.data_ptr(), ctypes.c_float(1e-5), hd.data_ptr(), y,
                                                        n, k, m, batch, ctypes.byref(st), hs)
                return lib.row_exact_mv(t, wp[i % copies], xd.data_ptr(), y, n, k, m, batch, ctypes.byref(st), hs)

            for tag in libs:
                with torch.cuda.stream(stream):
                    rc = run(tag, 0)
                torch.cuda.synchronize()
                if rc:
                    raise RuntimeError(f"{name} m={m}: build {tag} returned {rc}")
            same = torch.equal(ys["a"].view(torch.int32), ys["b"].view(torch.int32))
            reps = int(min(200, max(30, 3e-3 / (w.weight_bytes / 2.5e12))))
            times = {tag: [] for tag in libs}
            for r in range(5):
                for tag in libs:
                    with torch.cuda.stream(stream):
                        for i in range(3):
                            run(tag, i)
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        torch.cuda._sleep(int(2e6))
                        e0.record(stream)
                        for i in range(reps):
                            run(tag, i + r)
                        e1.record(stream)
                    torch.cuda.synchronize()
                    times[tag].append(e0.elapsed_time(e1) * 1e3 / reps)
            a, b = statistics.median(times["a"]), statistics.median(times["b"])
            rec = {"workload": name, "m": m, "a_us": round(a, 3), "b_us": round(b, 3), "b_over_a": round(b / a, 4),
                   "bitwise_same": bool(same),
                   "max_abs_diff": float((ys["a"] - ys["b"]).abs().max().item()),
                   "a_schedule": qfr.row_exact_schedule(t, n, k, m, batch).asdict()}
            res.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
        del Wd
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump({"a": os.path.relpath(qfr._LIB_PATH, ROOT), "b": other_path, "results": res}, f, indent=1)


if __name__ == "__main__":
    main()
