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
measured with HIP events recorded on the sort's stream around every launch,
in a second timed region (the headline number is timed without those
events).
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


def cpu_baseline(keys, values, begin_bit, end_bit, budget_s=12.0):
    import oracle
    n = keys.size
    m = min(n, 1 << 26)
    ks = np.ascontiguousarray(keys[:m])
    vs = None if values is None else np.ascontiguousarray(values[:m])
    runs, total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.lsd_sort(ks, vs, begin_bit, end_bit, RADIX_BITS)
        total += time.perf_counter() - t0
        runs += 1
        if total >= budget_s or runs >= 20:
            break
    rate = m * runs / total / 1e9
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(rate, 5), "unit": "Gkeys/s", "cores": 1, "kind": "oracle",
        "cpu_model": model, "host_cores": os.cpu_count(),
        "sample": f"first {m} keys of the workload, {runs} run(s), {total:.1f} s total, "
                  f"single-threaded counting-sort LSD (r={RADIX_BITS})",
    }


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

    # Per-kernel durations: second timed region with an event pair around
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--write-traffic-profile", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/pass_kernel_traffic_<workload>.md from rocprofv3 csv dirs")
    ap.add_argument("--profile-command", default="", help="command line recorded with --write-traffic-profile")
    args = ap.parse_args(argv)

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
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        record["cpu_baseline"] = cpu_baseline(keys, values, b, e)
    print(json.dumps(record), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
