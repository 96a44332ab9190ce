#!/usr/bin/env python3
"""Benchmark of the gfx950 stable LSD radix sort on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

One step = one complete sort call (all digit passes plus the histogram,
scan and fill kernels) over the workload's keys, which are resident in device
memory before timing starts; the input buffer is never modified (out of
place), so every step sorts the same data.  Prints ONE JSON line on stdout.

Default workload: 2^28 uniform uint32 keys, keys only (the 1 GiB large-N
configuration; the sort is HBM-bound there and its data does not fit in the
last-level cache).  Other workloads: see lsd_radix_sort_pass_amd.workloads;
"morton_points_2^24" times the Morton-code sort of 2^24 float32 points
(codes computed where the points are read, sorted with point indices).

roofline: the dominant kernel is the one with the largest time per sort,
normally the digit pass (rank + chained scan + scatter).  A pass's
algorithmic bytes are n * 2 * (key bytes + value bytes): every key and value
read and written once.  Passes the library skipped (one digit for every key,
or keys already in order) move nothing, so a pass launch is credited with
the executed passes' bytes averaged over the launches (one copy's worth when
no pass ran); the histogram kernel reads n * key bytes.  Durations are
measured with a pair of HIP events attached to every kernel's dispatch on
the sort's stream (hipExtLaunchKernel: they stamp the kernel's own start
and end, as a profiler's kernel trace does), in a second timed region (the
headline number is timed without those events).
traffic: HBM bytes per pass launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
counters, scaled by the same counters read on a plain copy of known size,
read from profiles/ when they were taken on the current kernel source
(else null).
cpu_baseline: the CPU oracle (single-threaded counting-sort LSD) timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
DEFAULT_WORKLOAD = "uniform_u32_2^28"
RADIX_BITS = 8                  # digit width of the library's pass plan
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "lsd_radix_sort_pass_amd", "csrc")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per pass launch recorded under profiles/ for this workload,
    if they were measured on the current kernel source."""
    path = os.path.join(PROFILES, f"pass_kernel_traffic_{workload.replace('^', '')}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^kernel_source_hash:\s*(\w+)", text, flags=re.M)
    m_bytes = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, flags=re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def _median_rate(fn, m, runs_max, budget_s):
    """Median keys/s of up to runs_max timed calls of fn (at least 3, fewer
    than runs_max once budget_s is spent)."""
    times = []
    while len(times) < runs_max:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and sum(times) >= budget_s:
            break
    times.sort()
    return m / times[len(times) // 2] / 1e9, len(times), sum(times)


def cpu_baseline(keys, values, begin_bit, end_bit, budget_s=8.0):
    """The oracle (single-threaded counting-sort LSD) timed on the host: the
    median over runs on a 2^26-key sample of the workload.  As context, for
    uint32/int32 keys-only workloads, std::sort and std::stable_sort on one
    core (the comparison sorts [SS] "測定" timed) on a 2^24-key sample."""
    import oracle
    n = keys.size
    m = min(n, 1 << 26)
    ks = np.ascontiguousarray(keys[:m])
    vs = None if values is None else np.ascontiguousarray(values[:m])
    rate, runs, total = _median_rate(lambda: oracle.lsd_sort(ks, vs, begin_bit, end_bit, RADIX_BITS),
                                     m, 7, budget_s)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    record = {
        "value": round(rate, 5), "unit": "Gkeys/s", "cores": 1, "kind": "oracle",
        "cpu_model": model, "host_cores": os.cpu_count(),
        "sample": f"first {m} keys of the workload, median of {runs} run(s) ({total:.1f} s in all), "
                  f"single-threaded counting-sort LSD (r={RADIX_BITS})",
    }
    if values is None and keys.dtype in (np.dtype(np.uint32), np.dtype(np.int32)) and (begin_bit, end_bit) == (0, 32):
        mc = min(n, 1 << 24)
        kc = np.ascontiguousarray(keys[:mc])
        ctx = {}
        for name, stable in (("std_sort", False), ("std_stable_sort", True)):
            r, runs_c, _ = _median_rate(lambda: oracle.std_sort(kc, stable), mc, 3, 0.0)
            ctx[name] = round(r, 5)
        ctx["unit"] = "Gkeys/s"
        ctx["cores"] = 1
        ctx["sample"] = f"first {mc} keys, native {keys.dtype.name} order, median of 3 runs each"
        record["context"] = ctx
    return record


COPY_WORDS = 1 << 28            # calibration copy: 1 GiB read + 1 GiB written


def run_copy_calibration(steps: int) -> int:
    """A plain device copy of known size, run under rocprofv3 --pmc to turn
    FETCH_SIZE / WRITE_SIZE readings into bytes."""
    import torch
    import lsd_radix_sort_pass_amd as rs
    a = torch.zeros(COPY_WORDS, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(steps):
        rs.copy_u32(a, b)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {steps} copies of {COPY_WORDS} words")
    return 0


def _pmc_mean_kib(run_dir: str, kernel_substr: str, counter: str) -> float:
    """Mean per-dispatch value of `counter` for kernels whose name contains
    `kernel_substr`, from a rocprofv3 --output-format csv directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals = []
    for f in files:
        for row in csv.DictReader(open(f)):
            if kernel_substr in row["Kernel_Name"] and row["Counter_Name"] == counter:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} samples for '{kernel_substr}' under {run_dir}")
    return sum(vals) / len(vals)


def write_traffic_profile(workload: str, fetch_dir: str, write_dir: str,
                          copy_fetch_dir: str, copy_write_dir: str, command: str) -> str:
    """Turn FETCH_SIZE / WRITE_SIZE readings (KiB per dispatch) of the pass
    kernel into HBM bytes per launch, scaled by what the same counters read
    for the calibration copy (which moves exactly COPY_WORDS*4 bytes each
    way), and record them under profiles/ with the kernel source hash."""
    copy_bytes = COPY_WORDS * 4
    cf = _pmc_mean_kib(copy_fetch_dir, "copy_u128_kernel", "FETCH_SIZE")
    cw = _pmc_mean_kib(copy_write_dir, "copy_u128_kernel", "WRITE_SIZE")
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    pf = _pmc_mean_kib(fetch_dir, "onesweep_kernel", "FETCH_SIZE")
    pw = _pmc_mean_kib(write_dir, "onesweep_kernel", "WRITE_SIZE")
    hf = _pmc_mean_kib(fetch_dir, "hist_kernel", "FETCH_SIZE")
    fetch_bytes = pf * 1024.0 * fetch_scale
    write_bytes = pw * 1024.0 * write_scale
    w = __import__("lsd_radix_sort_pass_amd.workloads", fromlist=["WORKLOADS"]).WORKLOADS[workload]
    word = 8 if w.pairs else 4
    algo = 2 * word * w.n
    path = os.path.join(PROFILES, f"pass_kernel_traffic_{workload.replace('^', '')}.md")
    with open(path, "w") as f:
        f.write(f"# HBM traffic of the digit-pass kernel, workload {workload}\n\n")
        f.write("Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (separate runs),\n"
                "KiB per dispatch, mean over the pass-kernel dispatches.  Scaled by the same\n"
                f"counters read on a plain copy of {copy_bytes} bytes each way.\n\n")
        f.write(f"command: {command}\n\n")
        f.write(f"copy FETCH_SIZE KiB: {cf:.1f} -> fetch scale {fetch_scale:.4f}\n")
        f.write(f"copy WRITE_SIZE KiB: {cw:.1f} -> write scale {write_scale:.4f}\n")
        f.write(f"pass FETCH_SIZE KiB: {pf:.1f} -> {fetch_bytes:.4g} bytes\n")
        f.write(f"pass WRITE_SIZE KiB: {pw:.1f} -> {write_bytes:.4g} bytes\n")
        f.write(f"hist FETCH_SIZE KiB: {hf:.1f} -> {hf * 1024.0 * fetch_scale:.4g} bytes (reads n*4 = {4 * w.n})\n")
        f.write(f"algorithmic bytes per pass launch: {algo}\n")
        f.write(f"traffic / algorithmic: {(fetch_bytes + write_bytes) / algo:.3f}\n\n")
        f.write(f"traffic_bytes_per_launch: {fetch_bytes + write_bytes:.6g}\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
    return path


def _csv_rows(run_dir: str, suffix: str):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {run_dir}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _short_name(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def _pass_dispatches(rows, warmup: int, passes: int):
    """The pass-kernel dispatches of the timed sorts, in launch order, each
    with its pass index (every sort launches one pass kernel per pass, so
    index = launch number mod passes); the first `warmup` sorts are dropped."""
    ps = [r for r in rows if "onesweep_kernel" in r["Kernel_Name"]]
    ps.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
    ps = ps[warmup * passes:]
    return [(i % passes, r) for i, r in enumerate(ps)]


def _bench_record(path: str) -> dict:
    lines = [ln for ln in open(path) if ln.lstrip().startswith("{")]
    if not lines:
        raise ValueError(f"no bench JSON line in {path}")
    return json.loads(lines[-1])


def write_kernel_stats(run_dir: str, bench_log: str, command: str, warmup: int) -> str:
    """Summarise a rocprofv3 --kernel-trace --stats run of bench.py under
    profiles/: every kernel over all dispatches, then the pass kernel per
    pass index over the timed sorts (warmup dropped), with each index's
    fraction of the HBM peak from its algorithmic bytes."""
    rec = _bench_record(bench_log)
    cfg = rec["config"]
    workload, n, passes = cfg["workload"], cfg["n"], cfg["passes"]
    rows = _csv_rows(run_dir, "kernel_trace.csv")
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    by_name = {}
    for r in rows:
        by_name.setdefault(r["Kernel_Name"], []).append(dur(r))
    total_all = sum(sum(v) for v in by_name.values())
    skipped = {x["pass"] for x in rec.get("kernels", {}).get("pass_by_index", []) if x.get("skipped")}
    if workload.startswith("morton_points"):
        word_bytes = {0: 20 * n}
        bytes_of = lambda p: word_bytes.get(p, 16 * n)
    else:
        w = __import__("lsd_radix_sort_pass_amd.workloads", fromlist=["WORKLOADS"]).WORKLOADS[workload]
        word = np.dtype(w.dtype).itemsize + (np.dtype(w.value_dtype).itemsize if w.pairs else 0)
        bytes_of = lambda p: 2 * word * n
    per = {}
    for p, r in _pass_dispatches(rows, warmup, passes):
        per.setdefault(p, []).append(dur(r))
    prefix = {"all-pass digit histogram": "hist_kernel", "one-launch sort (all passes)": "small_sort_kernel"}.get(
        rec["roofline"]["kernel"], "pass_kernel")
    path = os.path.join(PROFILES, f"{prefix}_{workload.replace('^', '')}_kernel_stats.md")
    with open(path, "w") as f:
        f.write(f"# Kernel durations: {workload} sort ({cfg.get('description', '')})\n\n")
        f.write("command (from the repository root, on one MI355X):\n\n")
        f.write(f"    {command}\n\n")
        f.write("rocprofv3 kernel trace, all dispatches of the run (warmup included; ns):\n\n")
        f.write("| kernel | calls | total ns | average ns | min ns | max ns | % |\n|---|---|---|---|---|---|---|\n")
        for name, v in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
            f.write(f"| `{_short_name(name)}` | {len(v)} | {sum(v)} | {sum(v) // len(v)} | {min(v)} | {max(v)} | "
                    f"{100.0 * sum(v) / total_all:.2f} |\n")
        f.write(f"\nPass kernel per pass index over the timed sorts (first {warmup} sorts dropped; "
                f"{n} keys; a pass's algorithmic bytes are n x 2 x (key + value bytes) = {bytes_of(1)}):\n\n")
        f.write("| pass | dispatches | average ns | median ns | min ns | max ns | frac of 8 TB/s (average) "
                "| frac (median) | frac (slowest) |\n|---|---|---|---|---|---|---|---|---|\n")
        for p in sorted(per):
            v = sorted(per[p])
            avg = sum(v) / len(v)
            med = v[len(v) // 2]
            if p in skipped:
                f.write(f"| {p} | {len(v)} | {avg:.0f} | {med} | {v[0]} | {v[-1]} | skipped | skipped | skipped |\n")
                continue
            fr = lambda t: bytes_of(p) / (t * 1e-9) / 1e9 / HBM_PEAK_GBS
            f.write(f"| {p} | {len(v)} | {avg:.0f} | {med} | {v[0]} | {v[-1]} | {fr(avg):.3f} | {fr(med):.3f} "
                    f"| {fr(v[-1]):.3f} |\n")
        f.write("\nbench.py line of the same run:\n\n")
        f.write("    " + json.dumps({k: rec[k] for k in ("value", "unit", "ms_per_step", "roofline", "kernels")
                                     if k in rec}) + "\n")
        f.write(f"\nkernel_source_hash: {kernel_source_hash()}\n")
    return path


def write_counter_profile(run_dirs, bench_log: str, command: str, warmup: int, tag: str,
                          kernel: str = "onesweep_kernel") -> str:
    """Summarise rocprofv3 --pmc runs of bench.py under profiles/: the mean
    of every counter per dispatch of the pass kernel, per pass index over
    the timed sorts (or, for kernel="hist_kernel", of the histogram kernel,
    one dispatch per sort), plus derived shares (LDS bank-conflict cycles of
    LDS active cycles, waves' waiting share)."""
    rec = _bench_record(bench_log)
    cfg = rec["config"]
    workload = cfg["workload"]
    passes = cfg["passes"] if kernel == "onesweep_kernel" else 1
    table = {}
    for d in run_dirs:
        rows = _csv_rows(d, "counter_collection.csv")
        per_dispatch = {}
        for r in rows:
            if kernel not in r["Kernel_Name"]:
                continue
            key = int(r["Dispatch_Id"])
            per_dispatch.setdefault(key, {})
            c = r["Counter_Name"]
            per_dispatch[key][c] = per_dispatch[key].get(c, 0.0) + float(r["Counter_Value"])
        ids = sorted(per_dispatch)[warmup * passes:]
        for i, key in enumerate(ids):
            p = i % passes
            for c, v in per_dispatch[key].items():
                table.setdefault(c, {}).setdefault(p, []).append(v)
    name = "pass_kernel" if kernel == "onesweep_kernel" else kernel
    path = os.path.join(PROFILES, f"{name}_counters_{workload.replace('^', '')}{tag}.md")
    mean = lambda c, p: sum(table[c][p]) / len(table[c][p])
    with open(path, "w") as f:
        what = "the digit-pass kernel per pass index" if kernel == "onesweep_kernel" else f"`{kernel}`"
        f.write(f"# Hardware counters of {what}, workload {workload}\n\n")
        f.write("commands (from the repository root, one MI355X; each counter set a run of its own):\n\n")
        for c in command.split(" ;; "):
            f.write(f"    {c}\n")
        f.write(f"\nMean per dispatch over the timed sorts (first {warmup} sorts dropped):\n\n")
        idx = sorted({p for c in table for p in table[c]})
        label = (lambda p: f"pass {p}") if kernel == "onesweep_kernel" else (lambda p: "per dispatch")
        f.write("| counter | " + " | ".join(label(p) for p in idx) + " |\n")
        f.write("|---|" + "---|" * len(idx) + "\n")
        for c in sorted(table):
            f.write(f"| {c} | " + " | ".join(f"{mean(c, p):.4g}" for p in idx) + " |\n")
        derived = []
        if "SQ_LDS_BANK_CONFLICT" in table and "SQ_LDS_IDX_ACTIVE" in table:
            derived.append(("LDS bank-conflict cycles / LDS indexed-active cycles",
                            [mean("SQ_LDS_BANK_CONFLICT", p) / max(mean("SQ_LDS_IDX_ACTIVE", p), 1) for p in idx]))
        if "SQ_LDS_ADDR_CONFLICT" in table and "SQ_LDS_IDX_ACTIVE" in table:
            derived.append(("LDS same-address conflict cycles / LDS indexed-active cycles",
                            [mean("SQ_LDS_ADDR_CONFLICT", p) / max(mean("SQ_LDS_IDX_ACTIVE", p), 1) for p in idx]))
        if "SQ_WAIT_INST_LDS" in table and "SQ_WAVE_CYCLES" in table:
            derived.append(("waves waiting to issue an LDS instruction / wave cycles",
                            [mean("SQ_WAIT_INST_LDS", p) / max(mean("SQ_WAVE_CYCLES", p), 1) for p in idx]))
        if "SQ_WAIT_ANY" in table and "SQ_WAVE_CYCLES" in table:
            derived.append(("waves waiting (any) / wave cycles",
                            [mean("SQ_WAIT_ANY", p) / max(mean("SQ_WAVE_CYCLES", p), 1) for p in idx]))
        if derived:
            f.write("\nDerived:\n\n| share | " + " | ".join(label(p) for p in idx) + " |\n")
            f.write("|---|" + "---|" * len(idx) + "\n")
            for name, vals in derived:
                f.write(f"| {name} | " + " | ".join(f"{v:.3f}" for v in vals) + " |\n")
        f.write(f"\nkernel_source_hash: {kernel_source_hash()}\n")
    return path


def time_steps(step, n, temp, args, torch, rs, _lib, dev):
    """Warm up, time args.steps calls of `step` (wall clock, bracketed by
    device synchronisation), then time them again with per-kernel events.
    Returns (Gkeys/s, ms per step, event ms over the first region, kernels)."""
    stream = torch.cuda.current_stream(dev)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    if rs.error_word(temp) != 0:
        raise RuntimeError("device guard word set after warmup")

    log(f"[bench] timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_events = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = n * args.steps / wall / 1e9

    # Per-kernel durations: second timed region with an event pair on
    # every launch, recorded on the sort's stream.
    rs.prof_reset()
    rs.prof_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    rs.prof_enable(False)
    kernels = {}
    for name, kind in [("fill", _lib.RS_KERNEL_FILL), ("hist", _lib.RS_KERNEL_HIST),
                       ("scan", _lib.RS_KERNEL_SCAN), ("pass", _lib.RS_KERNEL_PASS),
                       ("copy", _lib.RS_KERNEL_COPY), ("small", _lib.RS_KERNEL_SMALL)]:
        launches, ms = rs.prof_summary(kind)
        if launches:
            kernels[name] = {"launches": launches, "avg_us": round(ms * 1e3 / launches, 2)}
    # Per pass index: the median launch duration over the timed steps
    # (warmup excluded: the event region starts after it).
    by_index = []
    for p in range(8):
        samples = rs.prof_samples(_lib.RS_KERNEL_PASS, p)
        if not samples:
            break
        by_index.append({"pass": p, "launches": len(samples),
                         "median_us": round(float(np.median(samples)) * 1e3, 2),
                         "min_us": round(min(samples) * 1e3, 2), "max_us": round(max(samples) * 1e3, 2)})
    if by_index:
        kernels["pass_by_index"] = by_index
    rs.prof_reset()
    if rs.error_word(temp) != 0:
        raise RuntimeError("device guard word set after timing")
    return value, ms_per_step, ms_events, kernels


def bench_points(args, torch, rs, _lib, workloads, dev) -> int:
    """Morton-code sort of float32 points (rs_sort_morton30): codes computed
    where the points are read, sorted with point indices over 30 bits."""
    n = workloads.POINTS_WORKLOAD_N
    log(f"[bench] generating {args.workload} (n={n})")
    pts = workloads.make_points(n)
    dp = torch.from_numpy(pts).to(dev)
    codes = torch.empty(n, dtype=torch.uint32, device=dev)
    index = torch.empty(n, dtype=torch.uint32, device=dev)
    temp = torch.empty(rs.temp_bytes_morton30(n), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize(dev)

    def step():
        rs.sort_morton30(dp, codes_out=codes, index_out=index, temp=temp)

    value, ms_per_step, ms_events, kernels = time_steps(step, n, temp, args, torch, rs, _lib, dev)
    # Algorithmic bytes: the first pass reads 12 B of point and writes 8 B
    # (code, index); the other three read and write 8 + 8 B.  Per launch:
    # the average over the four.
    passes = 4
    pass_bytes = (20 + 16 * (passes - 1)) * n // passes
    achieved = pass_bytes / (kernels["pass"]["avg_us"] * 1e-6) / 1e9
    kernels["pass"]["GBps"] = round(achieved, 1)
    kernels["hist"]["GBps"] = round(12 * n / (kernels["hist"]["avg_us"] * 1e-6) / 1e9, 1)
    record = {
        "metric": "Gkeys/s sorted (u32/f32 keys, 2^24-2^28, 1 GPU) + achieved HBM GB/s vs peak",
        "value": round(value, 3),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 points -> u32 Morton codes (single-precision quantisation, integer sort)",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": "2^24 float32 points uniform in the unit cube -> sorted 30-bit Morton codes + point indices",
            "n": n,
            "pairs": True,
            "begin_bit": 0,
            "end_bit": 30,
            "radix_bits": RADIX_BITS,
            "passes": passes,
            "event_ms_per_step": round(ms_events / args.steps, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "onesweep digit pass (first pass from points)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": pass_bytes,
        },
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] CPU baseline (oracle)")
        m = min(n, 1 << 24)
        sample = np.ascontiguousarray(pts[:m])
        runs, total = 0, 0.0
        while True:
            t0 = time.perf_counter()
            c = oracle.morton30(sample)
            oracle.lsd_sort(c, np.arange(m, dtype=np.uint32), 0, 30, RADIX_BITS)
            total += time.perf_counter() - t0
            runs += 1
            if total >= 12.0 or runs >= 20:
                break
        record["cpu_baseline"] = {
            "value": round(m * runs / total / 1e9, 5), "unit": "Gkeys/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} points, {runs} run(s), {total:.1f} s total, single-threaded Morton codes + "
                      f"counting-sort LSD (r={RADIX_BITS})",
        }
    print(json.dumps(record), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ranker", choices=["atomic", "match"], default="atomic",
                    help="local ranker of the digit passes (match: the ballot match ranker, 32-bit keys)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--write-traffic-profile", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/pass_kernel_traffic_<workload>.md from rocprofv3 csv dirs")
    ap.add_argument("--profile-command", default="", help="command line recorded with --write-* summaries")
    ap.add_argument("--write-kernel-stats", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="write profiles/pass_kernel_<workload>_kernel_stats.md from a rocprofv3 "
                         "--kernel-trace csv dir and the bench log of the same run")
    ap.add_argument("--write-counters", nargs="+", metavar="DIR",
                    help="BENCH_LOG then rocprofv3 --pmc csv dirs: write "
                         "profiles/pass_kernel_counters_<workload><tag>.md")
    ap.add_argument("--counters-tag", default="", help="file-name suffix for --write-counters")
    ap.add_argument("--counters-kernel", default="onesweep_kernel",
                    help="kernel whose dispatches --write-counters summarises (onesweep_kernel or hist_kernel)")
    args = ap.parse_args(argv)

    if args.write_kernel_stats:
        print(write_kernel_stats(*args.write_kernel_stats, command=args.profile_command, warmup=args.warmup))
        return 0
    if args.write_counters:
        print(write_counter_profile(args.write_counters[1:], args.write_counters[0], args.profile_command,
                                    args.warmup, args.counters_tag, args.counters_kernel))
        return 0
    if args.write_traffic_profile:
        print(write_traffic_profile(args.workload, *args.write_traffic_profile, command=args.profile_command))
        return 0
    if args.copy_calibration:
        return run_copy_calibration(max(args.steps, 1))

    if args.gpus != 1:
        print(f"bench.py: the sort runs on one GPU only (got --gpus {args.gpus}); "
              "it is a single-GPU kernel pipeline", file=sys.stderr)
        return 2

    import torch
    import lsd_radix_sort_pass_amd as rs
    from lsd_radix_sort_pass_amd import workloads, _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rs.prof_ranker(1 if args.ranker == "match" else 0)
    if args.workload == workloads.POINTS_WORKLOAD:
        return bench_points(args, torch, rs, _lib, workloads, dev)
    w = workloads.WORKLOADS[args.workload]
    log(f"[bench] generating {args.workload} (n={w.n})")
    keys, values, b, e = workloads.make(args.workload)
    n = keys.size
    dk = torch.from_numpy(keys).to(dev)
    dv = torch.from_numpy(values).to(dev) if values is not None else None
    ko = torch.empty_like(dk)
    vo = torch.empty_like(dv) if dv is not None else None
    kb = keys.dtype.itemsize
    vb = values.dtype.itemsize if values is not None else 0
    temp = rs.alloc_temp(n, dv is not None, b, e, device=dev, key_dtype=dk.dtype, value_bytes=vb or 4)
    torch.cuda.synchronize(dev)

    def step():
        if dv is None:
            rs.sort_keys(dk, b, e, out=ko, temp=temp)
        else:
            rs.sort_pairs(dk, dv, b, e, keys_out=ko, values_out=vo, temp=temp)

    value, ms_per_step, ms_events, kernels = time_steps(step, n, temp, args, torch, rs, _lib, dev)

    word = kb + vb                                  # bytes per key moved by a pass
    passes = (e - b + RADIX_BITS - 1) // RADIX_BITS
    hist_bytes = kb * n
    if "pass" in kernels:
        # A pass the library skipped (its digit is the same for every key, or
        # the keys were already in order) moves nothing; the output must still
        # be written once, so with no executed pass one copy is counted.
        skipped = rs.skipped_passes(temp, passes)
        executed = passes - sum(1 for f in skipped if f)
        pass_bytes = max(executed, 1) * 2 * word * n // passes    # average per pass launch
        candidates = {"pass": pass_bytes, "hist": hist_bytes}
    else:
        # Small inputs: the whole sort is one launch that reads and writes
        # the keys (and values) once per pass.
        executed = passes
        candidates = {"small": passes * 2 * word * n}
    for k, nb in candidates.items():
        kernels[k]["GBps"] = round(nb / (kernels[k]["avg_us"] * 1e-6) / 1e9, 1)
    pass_fracs = None
    if "pass_by_index" in kernels:
        # An executed pass reads and writes every key (and value) once; a
        # skipped one moves nothing and gets no fraction.
        flags = rs.skipped_passes(temp, passes)
        pass_fracs = []
        for rec in kernels["pass_by_index"]:
            if flags[rec["pass"]]:
                rec["skipped"] = True
                continue
            gbps = 2 * word * n / (rec["median_us"] * 1e-6) / 1e9
            rec["GBps"] = round(gbps, 1)
            rec["frac"] = round(gbps / HBM_PEAK_GBS, 4)
            pass_fracs.append(rec["frac"])
    # Dominant kernel: the one with the largest total time per step.
    dominant = max(candidates, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    kernel_name = {"pass": "onesweep digit pass", "hist": "all-pass digit histogram",
                   "small": "one-launch sort (all passes)"}[dominant]
    dom_bytes = candidates[dominant]
    achieved = dom_bytes / (kernels[dominant]["avg_us"] * 1e-6) / 1e9
    traffic = stored_traffic(args.workload) if dominant == "pass" else None
    dtype = f"{keys.dtype.kind}{8 * kb} keys" + (f" + {8 * vb}-bit values" if vb else "") + " (integer ops only)"

    record = {
        "metric": "Gkeys/s sorted (u32/f32 keys, 2^24-2^28, 1 GPU) + achieved HBM GB/s vs peak",
        "value": round(value, 3),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": w.description,
            "n": n,
            "pairs": dv is not None,
            "begin_bit": b,
            "end_bit": e,
            "radix_bits": RADIX_BITS,
            "passes": passes,
            "executed_passes": executed,
            "ranker": args.ranker,
            "event_ms_per_step": round(ms_events / args.steps, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
        },
        "kernels": kernels,
    }
    if pass_fracs:
        # Each executed pass on its own (median launch): the lowest fraction
        # and the fraction of every executed pass in pass order.
        record["roofline"]["pass_frac_min"] = min(pass_fracs)
        record["roofline"]["pass_frac_by_index"] = pass_fracs
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        record["cpu_baseline"] = cpu_baseline(keys, values, b, e)
    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
