"""Benchmark of overlap-save FIR filtering on one MI355X.

One step = one pass of the whole hot path over one batch of a workload.
The headline workload (default cfg4) is the largest configuration that fits
one GPU: M=16385 taps given as their 65536-point frequency response, L=49152,
5120 blocks (251,658,240 complex64 samples) in one call.  Before it, every
other configuration (cfg1, cfg2 with its 4 calls carrying the state, cfg3,
cfg5 with 1024 channels) is timed with its own warm-up, a sampled parity
check and a short oracle baseline, and reported under "configs".  Inputs
are resident in device memory before timing; a step rotates through enough
input/output buffer sets to exceed the 256 MB last-level cache, so every
step streams from HBM.

Prints one JSON line: Msamples/s of filtered output, the roofline of the
dominant kernel (algorithmic 16 B per sample: one complex64 read and one
write, timed with HIP events around the launches on the launch stream), a
copy reference, a parity check of one step against the float64 oracle and
the oracle's own CPU throughput (reported baseline, not a target).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, AMD published figure
VALU_PEAK_TFLOPS = 157.3          # MI355X fp32 vector, AMD published figure (packed fp32)
VALU_PEAK_UNPACKED_TFLOPS = 78.6  # 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz
# one rocprofv3 --pmc pass (7 SQ counters; at most 8 fit one pass)
VALU_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32 "
                 "SQ_INSTS_VALU_FMA_F32 SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES SQ_WAVES")
BYTES_PER_SAMPLE = 16             # complex64 in + complex64 out
LLC_BYTES = 256 << 20             # MI355X Infinity Cache
PROFILES_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: about one second of steps, at least 50)")
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed warm-up steps (default: about one second of steps)")
    ap.add_argument("--workload", default="cfg4",
                    help="headline workload: cfg1..cfg5 (default cfg4: M=16385, N=65536 "
                         "via H, 251658240 samples, the largest configuration), or a "
                         "channelizer workload (pfb1024, pfb128) measured alone")
    ap.add_argument("--no-table", action="store_true",
                    help="time the headline workload only (no per-configuration table); "
                         "for counter runs")
    ap.add_argument("--host-stream", action="store_true",
                    help="also time the host-resident streaming call (pinned host input "
                         "and output, copies overlapped with filtering); adds host_stream")
    ap.add_argument("--chunk", type=int, default=0,
                    help="samples per channel per step of the host-resident call (0: default)")
    ap.add_argument("--real", action="store_true",
                    help="also time real-valued input (two real rows per channel of the "
                         "workload, 8 B per real sample); adds real_pairs")
    ap.add_argument("--channelizer", default="", metavar="WORKLOAD",
                    help="also measure the polyphase channelizer on this workload "
                         "(pfb1024 or pfb128): adds a 'channelizer' object to the line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a profiles/ summary of a rocprofv3 --kernel-trace --stats "
                         "CSV run of this script, then exit")
    ap.add_argument("--trace-stdout", metavar="FILE", default="",
                    help="with --summarize-trace: the traced run's standard output; its "
                         "bench line gives each configuration's timed steps, and the "
                         "summary adds the mean of those dispatches")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="calibrate FETCH_SIZE / WRITE_SIZE runs of this script against "
                         "the copy kernel, write profiles/ summaries, then exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="tabulate FETCH_SIZE / WRITE_SIZE per dispatch of every filtering "
                         "kernel of a run with no copy kernel (e.g. tune_n.py), scaled by the "
                         "calibration stored in profiles/traffic.json")
    ap.add_argument("--summarize-valu", metavar="DIR",
                    help="write profiles/ VALU summaries of a rocprofv3 --pmc run of this "
                         "script with the counters of VALU_COUNTERS, then exit")
    ap.add_argument("--command", default="", help="command line recorded in the summary")
    ap.add_argument("--profiles-dir", default="",
                    help="where the summaries are written and read (default: profiles/)")
    return ap.parse_args()


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(files[0])))


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")[:80]


def _file_tag(kernel: str) -> str:
    """A kernel name as a file-name part: ols_fused_kernel<12, false> ->
    ols_fused_kernel_12_false."""
    k = kernel.split("::")[-1]
    return re.sub(r"[^A-Za-z0-9]+", "_", k).strip("_")


def _bench_line(path: str):
    """The last JSON bench line of a run's standard output, or None."""
    line = None
    for ln in open(path, errors="replace"):
        ln = ln.strip()
        if ln.startswith("{") and '"metric"' in ln:
            try:
                line = json.loads(ln)
            except ValueError:
                pass
    return line


def timed_dispatches(trace_dir: str, kernel: str, n: int):
    """Durations (us) of the last n dispatches of `kernel` (as _short prints
    it) in a rocprofv3 kernel trace: the timed region of the bench run that
    launched it last, since nothing launches a filtering kernel after its
    timed steps."""
    rows = [r for r in _csv_rows(trace_dir, "kernel_trace.csv")
            if _short(r["Kernel_Name"]) == kernel]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[-n:]]


def summarize_trace(args):
    """profiles/<kernel>_<workload>_kernel_trace.md from run_kernel_stats.csv:
    one summary per configuration whose filtering kernel the run launched
    (the default bench run launches all of them: the table and the
    headline), each listing that kernel's calls and durations."""
    import workloads as W
    rows = _csv_rows(args.summarize_trace, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    by_name = {_short(r["Name"]).split("::")[-1]: r for r in rows}
    line = _bench_line(args.trace_stdout) if args.trace_stdout else None
    keys = list(TABLE_KEYS) if args.workload in TABLE_KEYS else [args.workload]
    written = []
    for key in keys:
        if key not in W.WORKLOADS:
            # the channelizer and the multi-pass runs: the top kernel by GPU time
            r = rows[0]
        else:
            kern = roofline_kernel(W.WORKLOADS[key].N)
            r = by_name.get(kern)
            if r is None:
                continue
        name = _short(r["Name"])
        timed = []
        if line is not None:
            cfg = (line.get("configs") or {}).get(key)
            if cfg is None and key == args.workload:
                cfg = {"steps": line.get("steps"),
                       "calls_per_step": (line.get("config") or {}).get("calls_per_step"),
                       "avg_launch_us": (line.get("roofline") or {}).get("avg_launch_us")}
            if cfg and cfg.get("steps") and cfg.get("calls_per_step"):
                n = int(cfg["steps"]) * int(cfg["calls_per_step"])
                d = timed_dispatches(args.summarize_trace, name, n)
                if len(d) == n:
                    timed = [f"Timed region of the traced run: its last {n} dispatches "
                             f"({cfg['steps']} steps x {cfg['calls_per_step']} calls) average "
                             f"{np.mean(d):.3f} us (min {min(d):.3f}, max {max(d):.3f}); the "
                             f"bench line's avg_launch_us (HIP events around the same steps, "
                             f"gaps between launches included) is {cfg.get('avg_launch_us')}.",
                             ""]
        out = os.path.join(PROFILES_DIR, f"{_file_tag(name)}_{key}_kernel_trace.md")
        lines = [f"# Kernel trace: {key} ({WORKLOAD_NOTE.get(key, '')})", "",
                 "Command (working directory /tmp):", "", "```", args.command, "```", "",
                 f"Kernel source hash: `{kernel_source_hash(key)}`", "",
                 "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
                 "|---|---|---|---|---|---|",
                 f"| `{name}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                 f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | "
                 f"{float(r['Percentage']):.1f}% |", "",
                 "The average covers every dispatch of the run, warm-up and parity calls "
                 "included.", ""] + timed + [
                 "Other kernels of the same run (top 8 by GPU time):", "",
                 "| kernel | calls | average (us) | share of GPU time |", "|---|---|---|---|"]
        for o in rows[:8]:
            lines.append(f"| `{_short(o['Name'])}` | {o['Calls']} | "
                         f"{float(o['AverageNs'])/1e3:.3f} | {float(o['Percentage']):.1f}% |")
        open(out, "w").write("\n".join(lines) + "\n")
        written.append(out)
    for w in written:
        print(w)


def summarize_pmc(args):
    """Calibrated HBM traffic of the filtering kernel from two counter runs."""
    import workloads as W
    w = W.WORKLOADS[args.workload]
    copy_kib = w.nchan * w.samples * 8 / 1024.0   # bytes read (= written) by the copy kernel
    res = {}
    for counter, d in (("FETCH_SIZE", args.summarize_pmc[0]), ("WRITE_SIZE", args.summarize_pmc[1])):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        ols = {k: v for k, v in per.items() if "ols_" in k and "plan_taps" not in k}
        cal = [v for k, v in per.items() if "neg" in k]
        if not ols or not cal:
            raise SystemExit(f"{counter}: filtering or copy kernel missing in {d}")
        cal_mean = float(np.mean(cal[0]))
        scale = copy_kib / cal_mean
        res[counter] = {"scale": scale, "copy_kib_counted": cal_mean, "copy_kib_true": copy_kib,
                        "kernels": {_short(k): float(np.mean(v)) for k, v in ols.items()}}
    kernels = res["FETCH_SIZE"]["kernels"]
    calls = len(w.calls)
    step_bytes = 0.0
    for k in kernels:
        step_bytes += (kernels[k] * res["FETCH_SIZE"]["scale"]
                       + res["WRITE_SIZE"]["kernels"].get(k, 0.0) * res["WRITE_SIZE"]["scale"]) * 1024
    # per launch of the filtering call (all kernels of one call)
    per_launch = step_bytes  # counters are per dispatch; one dispatch per call
    alg = w.nchan * w.samples / calls * BYTES_PER_SAMPLE
    path = os.path.join(PROFILES_DIR, "traffic.json")
    try:
        db = json.load(open(path))
    except (OSError, ValueError):
        db = {}
    db[args.workload] = {"bytes_per_launch": round(per_launch), "algorithmic_bytes_per_launch": alg,
                         "ratio": round(per_launch / alg, 4),
                         "source_hash": kernel_source_hash(args.workload),
                         "fetch_scale": round(res["FETCH_SIZE"]["scale"], 4),
                         "write_scale": round(res["WRITE_SIZE"]["scale"], 4)}
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    top = _file_tag(sorted(kernels)[0])
    out = os.path.join(PROFILES_DIR, f"{top}_{args.workload}_hbm_traffic.md")
    lines = [f"# HBM traffic: {args.workload} ({WORKLOAD_NOTE.get(args.workload, '')})", "",
             "Two counter runs of the same command, one per counter (working directory /tmp):",
             "", "```", args.command, "```", "",
             f"Kernel source hash: `{kernel_source_hash(args.workload)}`", "",
             "The counters are read per dispatch in KiB.  Each is scaled by the ratio of the true "
             "bytes to the counted KiB of the elementwise copy kernel in the same run "
             f"(`torch.neg` over {copy_kib:.0f} KiB read and written).", "",
             "| counter | copy kernel counted (KiB) | true (KiB) | scale |", "|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"| {c} | {res[c]['copy_kib_counted']:.1f} | {copy_kib:.1f} | {res[c]['scale']:.4f} |")
    lines += ["", "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled bytes per dispatch |",
              "|---|---|---|---|"]
    for k in kernels:
        fb = kernels[k] * res["FETCH_SIZE"]["scale"] * 1024
        wb = res["WRITE_SIZE"]["kernels"].get(k, 0.0) * res["WRITE_SIZE"]["scale"] * 1024
        lines.append(f"| `{k}` | {kernels[k]:.1f} | {res['WRITE_SIZE']['kernels'].get(k, 0.0):.1f} | "
                     f"{fb + wb:.4g} |")
    lines += ["", f"Algorithmic bytes per call (16 B per output sample): {alg:.4g}.  "
              f"Measured / algorithmic: {per_launch / alg:.3f}."]
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_counters(args):
    """profiles/<kernel>_<workload>_hbm_counters.md: per-dispatch HBM
    counters of every filtering kernel, scaled by the counters' calibration
    on the copy kernel of the bench runs (fetch_scale / write_scale of the
    records in profiles/traffic.json)."""
    db = json.load(open(os.path.join(PROFILES_DIR, "traffic.json")))
    fs = float(np.median([r["fetch_scale"] for r in db.values()]))
    ws = float(np.median([r["write_scale"] for r in db.values()]))
    per = {}
    for counter, d in (("FETCH_SIZE", args.summarize_counters[0]),
                       ("WRITE_SIZE", args.summarize_counters[1])):
        for r in _csv_rows(d, "counter_collection.csv"):
            k = r["Kernel_Name"]
            if (r["Counter_Name"] == counter and ("ols_" in k or "pfb_" in k)
                    and "plan_taps" not in k):
                per.setdefault(_short(k), {}).setdefault(counter, []).append(
                    float(r["Counter_Value"]))
    if not per:
        raise SystemExit("no filtering kernel in the counter runs")
    top = _file_tag(max(per, key=lambda k: np.mean(per[k].get("FETCH_SIZE", [0.0]))))
    out = os.path.join(PROFILES_DIR, f"{top}_{args.workload}_hbm_counters.md")
    lines = [f"# HBM counters: {args.workload} ({WORKLOAD_NOTE.get(args.workload, '')})", "",
             "Two counter runs of the same command, one per counter (working directory /tmp):",
             "", "```", args.command, "```", "",
             f"Kernel source hash: `{kernel_source_hash(args.workload)}`", "",
             f"Mean KiB per dispatch; scaled bytes use FETCH_SIZE x {fs:.4g} and WRITE_SIZE x "
             f"{ws:.4g}, the counters' calibration on an elementwise copy of known size.", "",
             "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled MB per dispatch |",
             "|---|---|---|---|---|"]
    for k in sorted(per):
        f = float(np.mean(per[k].get("FETCH_SIZE", [0.0])))
        w_ = float(np.mean(per[k].get("WRITE_SIZE", [0.0])))
        lines.append(f"| `{k}` | {len(per[k].get('FETCH_SIZE', []))} | {f:.1f} | {w_:.1f} | "
                     f"{(f * fs + w_ * ws) * 1024 / 1e6:.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_valu(args):
    """VALU instruction and fp32 flop counts per dispatch of the filtering
    kernel, from one counter run; stored per workload in profiles/valu.json."""
    import workloads as W
    w = W.WORKLOADS[args.workload]
    per = {}
    for r in _csv_rows(args.summarize_valu, "counter_collection.csv"):
        k = r["Kernel_Name"]
        if "ols_" not in k or "plan_taps" in k:
            continue
        per.setdefault(_short(k), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"filtering kernel missing in {args.summarize_valu}")
    names = VALU_COUNTERS.split()
    kern = sorted(per)[0]
    mean = {c: float(np.mean(per[kern][c])) for c in names if c in per[kern]}
    missing = [c for c in names if c not in mean]
    if missing:
        raise SystemExit(f"counters missing: {missing}")
    # wave-level instruction counts; every lane of the kernels' waves is active
    flops = 64.0 * (mean["SQ_INSTS_VALU_ADD_F32"] + mean["SQ_INSTS_VALU_MUL_F32"]
                    + 2.0 * mean["SQ_INSTS_VALU_FMA_F32"])
    samples = w.nchan * w.samples / len(w.calls)
    rec = {"kernel": kern, "source_hash": kernel_source_hash(args.workload),
           "valu_instr_per_launch": mean["SQ_INSTS_VALU"],
           "fp32_flops_per_launch": flops,
           "valu_instr_per_sample": round(64.0 * mean["SQ_INSTS_VALU"] / samples, 2),
           "fp32_flops_per_sample": round(flops / samples, 2),
           "counters": {c: mean[c] for c in names}}
    path = os.path.join(PROFILES_DIR, "valu.json")
    try:
        db = json.load(open(path))
    except (OSError, ValueError):
        db = {}
    db[args.workload] = rec
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    top = _file_tag(kern)
    out = os.path.join(PROFILES_DIR, f"{top}_{args.workload}_valu.md")
    lines = [f"# VALU counters: {args.workload} ({WORKLOAD_NOTE.get(args.workload, '')})", "",
             "One counter run (working directory /tmp):", "", "```", args.command, "```", "",
             f"Kernel source hash: `{kernel_source_hash(args.workload)}`", "",
             f"Mean per dispatch of `{kern}` ({len(per[kern]['SQ_WAVES'])} dispatches):", "",
             "| counter | value |", "|---|---|"]
    for c in names:
        lines.append(f"| {c} | {mean[c]:.6g} |")
    lines += ["", f"fp32 flops per dispatch = 64 x (ADD_F32 + MUL_F32 + 2 FMA_F32) = {flops:.4g} "
              f"({flops / samples:.1f} per output sample; VALU lane-instructions per output "
              f"sample: {64.0 * mean['SQ_INSTS_VALU'] / samples:.1f}).  `bench.py` divides the "
              "flops by the live per-launch duration for the VALU line of its output."]
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def measured_valu(workload: str):
    """The counter record of profiles/valu.json if it was taken with the
    current kernel sources (else None)."""
    path = os.path.join(PROFILES_DIR, "valu.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(workload):
        return None
    return rec


def cpu_baseline(inp, seconds_budget: float = 20.0, single_seconds: float = 2.0):
    """Time the float64 oracle on the host cores on a bounded output sample.

    Returns the baseline record and the oracle outputs it computed (all
    outputs when the whole workload fits the budget, else None).
    """
    import oracle
    w = inp.workload
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(int(threads), 64))
    total = w.nchan * w.samples
    # calibrate on a small sample, then size the timed sample to the budget
    n_cal = 4096
    t0 = time.perf_counter()
    oracle.fir_direct(inp.h_ref, inp.x[0], inp.s0[0], idx=np.arange(min(n_cal, w.samples)),
                      threads=threads)
    per = (time.perf_counter() - t0) / min(n_cal, w.samples)
    want = int(min(total, max(n_cal, seconds_budget / max(per, 1e-12))))
    ref = None
    if want >= total:
        sample = f"all {total} outputs of the workload"
        reps, dt = 0, 0.0
        while reps < 100 and (reps == 0 or dt < 0.5 * seconds_budget):
            t0 = time.perf_counter()
            ref = oracle.fir_direct_multi(inp.h_ref, inp.x, inp.s0, threads=threads)
            dt += time.perf_counter() - t0
            reps += 1
        count = total * reps
        if reps > 1:
            sample += f", computed {reps} times"
    else:
        per_chan = max(1, want // w.nchan)
        idx = np.linspace(0, w.samples - 1, per_chan).astype(np.int64)
        sample = (f"{per_chan} evenly spaced outputs per channel x {w.nchan} channel(s) "
                  f"of {total}")
        t0 = time.perf_counter()
        oracle.fir_direct_multi(inp.h_ref, inp.x, inp.s0, idx=idx, threads=threads)
        dt = time.perf_counter() - t0
        count = per_chan * w.nchan
    # the same oracle on one thread, on a sample of about single_seconds
    n1 = int(max(256, min(w.samples, single_seconds / max(per * threads, 1e-12))))
    idx1 = np.linspace(0, w.samples - 1, n1).astype(np.int64)
    t0 = time.perf_counter()
    oracle.fir_direct(inp.h_ref, inp.x[0], inp.s0[0], idx=idx1, threads=1)
    dt1 = time.perf_counter() - t0
    return {"value": count / dt / 1e6, "unit": "Msamples/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3),
            "single_thread_value": n1 / dt1 / 1e6,
            "single_thread_sample": f"{n1} evenly spaced outputs of channel 0"}, ref


# Device sources each filtering path is compiled from (its kernel file and
# the headers that shape its device code; kernels.hpp only declares host
# functions); the counter records of a workload are keyed by the hash of
# its path's sources, so a change to another path's kernels leaves them
# valid.
COMMON_DEVICE_SOURCES = ("kernel_args.hpp", "geometry.hpp", "dft.hpp", "ols_phases.hpp",
                         "ols_block.hpp")
PATH_SOURCES = {
    "fused": ("ols_fused.hip",),
    "mid": ("ols_mid.hip", "ols_halfres.hpp"),
    "big": ("ols_big.hip", "ols_big.hpp"),
    "split": ("ols_split.hip", "ols_pair.hip", "ols_big.hpp"),
    "multi": ("ols_multi.hip", "ols_big.hpp"),
    "pfb": ("pfb.hip", "pfb.hpp"),
}


def kernel_path(N: int) -> str:
    """The filtering path of a plan with N-point blocks."""
    return ("fused" if N <= 8192 else "mid" if N == 16384 else "big" if N == 32768
            else "split" if N == 65536
            else "multi")


def kernel_source_hash(workload: str = "cfg2") -> str:
    """Hash of the device sources of the workload's filtering path, which
    its counter records are keyed by."""
    import hashlib

    import workloads as W
    w = W.WORKLOADS.get(workload)
    path = (kernel_path(w.N) if w is not None else
            "pfb" if workload in W.PFB_WORKLOADS else
            kernel_path(int(workload[1:])) if re.fullmatch(r"n\d+", workload) else "multi")
    d = os.path.join(ROOT, "order_fir_filtering_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(PATH_SOURCES[path] + COMMON_DEVICE_SOURCES):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken with the current kernel sources (else None)."""
    path = os.path.join(PROFILES_DIR, "traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def host_stream(args, inp, fo, torch, stream):
    """End-to-end rate of the host-resident streaming call on the same
    workload: input in pinned host memory, output back to pinned host memory,
    host-to-device copy, filtering and device-to-host copy pipelined by the
    library.  The host link bounds it; the plain pinned copy rates of the
    same bytes are reported beside it."""
    w = inp.workload
    sptr = stream.cuda_stream
    xh = torch.from_numpy(inp.x).pin_memory()
    yh = torch.empty(xh.shape, dtype=xh.dtype, pin_memory=True)
    plan = fo.Plan(w.M, w.N, w.nchan)
    if inp.H is not None:
        plan.set_freq_response(inp.H)
    else:
        plan.set_taps(inp.taps)
    plan.set_state(torch.from_numpy(inp.s0).to("cuda:0"))

    def hstep():
        pos = 0
        for c in w.calls:
            fo.fir_ols_execute_host(plan.handle, xh.data_ptr() + 8 * pos, yh.data_ptr() + 8 * pos,
                                    c, w.samples, args.chunk, sptr)
            pos += c

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        hstep()
    torch.cuda.synchronize()
    e0.record(stream)
    hstep()
    e1.record(stream)
    torch.cuda.synchronize()
    reps = max(3, min(200, int(1000.0 / max(e0.elapsed_time(e1), 1e-3))))
    e0.record(stream)
    for _ in range(reps):
        hstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    plan.close()
    # plain pinned copies of the same bytes, one direction at a time
    xd = torch.empty(xh.shape, dtype=xh.dtype, device="cuda:0")
    rates = {}
    for name, dst, src in (("h2d", xd, xh), ("d2h", yh, xd)):
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            dst.copy_(src, non_blocking=True)
        e1.record(stream)
        torch.cuda.synchronize()
        rates[name] = 5 * xh.numel() * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # both directions at once (the streaming call's situation), on two
    # default-priority streams
    s_in, s_out = torch.cuda.Stream(), torch.cuda.Stream()
    yd = torch.empty_like(xd)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        with torch.cuda.stream(s_in):
            xd.copy_(xh, non_blocking=True)
        with torch.cuda.stream(s_out):
            yh.copy_(yd, non_blocking=True)
    torch.cuda.synchronize()
    duplex = 5 * xh.numel() * 8 / (time.perf_counter() - t0) / 1e9
    samples = w.nchan * w.samples
    link = min(rates["h2d"], rates["d2h"]) * 1e9 / 8 / 1e6
    return {"value": round(samples / (ms * 1e-3) / 1e6, 1), "unit": "Msamples/s",
            "ms_per_step": round(ms, 4), "steps": reps, "pinned": True,
            "chunk": args.chunk or "default", "h2d_GBps": round(rates["h2d"], 1),
            "d2h_GBps": round(rates["d2h"], 1),
            "link_bound_Msamples": round(link, 1),
            "duplex_GBps_each_way": round(duplex, 1),
            "duplex_bound_Msamples": round(duplex * 1e9 / 8 / 1e6, 1),
            "note": "includes the host link; never the headline value"}


def real_pairs(inp, fo, torch, stream, nsets):
    """Real-valued input on the workload's shape: each complex channel
    becomes two real float32 rows of N(0,1) samples (seeded), filtered by
    the workload's real taps through fir_ols_execute_real, with the same
    calls per step.  Algorithmic bytes: 4 read + 4 written per real sample."""
    w = inp.workload
    if inp.taps is None:
        return {"skipped": "needs real taps"}
    rng = np.random.default_rng(20261202 + 100 + w.nchan)
    rows = torch.from_numpy(rng.standard_normal((2 * w.nchan, w.samples)).astype(np.float32))
    xs = [rows.to("cuda:0") for _ in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    sptr = stream.cuda_stream
    plan = fo.Plan(w.M, w.N, w.nchan)
    plan.set_taps(inp.taps)

    def rstep(k):
        x, y = xs[k % nsets], ys[k % nsets]
        pos = 0
        for c in w.calls:
            fo.fir_ols_execute_real(plan.handle, x.data_ptr() + 4 * pos, y.data_ptr() + 4 * pos,
                                    c, w.samples, sptr)
            pos += c

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k in range(5):
        rstep(k)
    torch.cuda.synchronize()
    e0.record(stream)
    rstep(0)
    e1.record(stream)
    torch.cuda.synchronize()
    reps = max(20, int(1000.0 / max(e0.elapsed_time(e1), 1e-3)))
    for k in range(reps):
        rstep(k)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(reps):
        rstep(k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    plan.close()
    samples = 2 * w.nchan * w.samples
    value = samples / (ms * 1e-3) / 1e6
    roof = HBM_PEAK_GBPS * 1e9 / 8 / 1e6
    return {"value": round(value, 1), "unit": "real Msamples/s", "ms_per_step": round(ms, 5),
            "steps": reps, "bytes_per_sample": 8, "roof_Msamples": roof,
            "hbm_roof_fraction": round(value / roof, 4),
            "rows": 2 * w.nchan, "samples_per_row": w.samples}


def channelizer(args, fo, torch, stream):
    """The polyphase channelizer on one of its workloads: parity of one call
    against the oracle on sampled output rows, then K timed calls of the
    whole input (the state and stream time carry from call to call), the
    per-launch rate against the HBM roof (8 B read per input sample, K/D
    outputs of 8 B written per hop of D samples), and the oracle timed on a
    bounded sample of rows."""
    import oracle
    import workloads as W
    key = args.channelizer
    w = W.PFB_WORKLOADS[key]
    K, D, Nh, n = w["K"], w["D"], w["Nh"], w["samples"]
    h, x_host = W.make_pfb_inputs(key)
    x = torch.from_numpy(x_host).to("cuda:0")
    y = torch.empty((n // D, K), dtype=torch.complex64, device="cuda:0")
    c = fo.Channelizer(K, D, Nh)
    c.set_taps(h)
    sptr = stream.cuda_stream
    out = {"workload": f"{key}: {w['description']}", "K": K, "D": D, "Nh": Nh,
           "samples_per_call": n, "outputs_per_call": n // D * K}
    # parity: the first call from zero state and time 0, sampled rows
    fo.fir_pfb_execute(c.handle, x, y, n, sptr)
    torch.cuda.synchronize()
    out["parity"] = None
    if not args.no_parity:
        rows = np.unique(np.concatenate([np.arange(16), W.sample_indices(11, n // D, 48),
                                         [n // D - 1]]))
        yg = y.cpu().numpy()[rows]
        ref = oracle.pfb_channelize(h, x_host, K, D, idx=rows)
        err = float(np.abs(yg.astype(np.complex128) - ref).max())
        bound = oracle.pfb_parity_bound(h, x_host)
        out["parity"] = {"max_abs_err": err, "bound": bound, "ok": err <= bound,
                         "rows_checked": int(rows.size), "outputs_checked": int(ref.size)}
    for _ in range(5):
        fo.fir_pfb_execute(c.handle, x, y, n, sptr)
    steps = args.steps if args.steps > 0 else 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fo.fir_pfb_execute(c.handle, x, y, n, sptr)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    c.close()
    byts = n * 8 + (n // D) * K * 8
    gbps = byts / (ms * 1e-3) / 1e9
    out.update({"metric": "channelized input Msamples/s (complex fp32)", "unit": "Msamples/s",
                "value": round(n / (ms * 1e-3) / 1e6, 1), "ms_per_call": round(ms, 4),
                "steps": steps,
                "roofline": {"bound": "hbm", "kernel": f"pfb_kernel<{int(np.log2(K))}, 8>",
                             "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(gbps / HBM_PEAK_GBPS, 4),
                             "algorithmic_bytes_per_launch": int(byts),
                             "bytes_per_input_sample": 8 + 8 * K / D}})
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):            # one core, BLAS included
            t0 = time.perf_counter()
            oracle.pfb_channelize(h, x_host, K, D, idx=np.arange(8))
            per = (time.perf_counter() - t0) / 8
            nrow = int(max(8, min(n // D, 15.0 / max(per, 1e-9))))
            t0 = time.perf_counter()
            oracle.pfb_channelize(h, x_host, K, D, idx=np.arange(nrow))
            sec = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(nrow * D / sec / 1e6, 4), "unit": "Msamples/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"first {nrow} output rows ({nrow * D} input "
                                         "samples), float64, one thread"}
    return out


def valu_line(workload: str, kern_ms: float):
    """fp32 VALU throughput of the filtering kernel: counted flops per
    launch (committed counter run of the same sources) over the live
    per-launch duration; None when the counters are stale."""
    rec = measured_valu(workload)
    if rec is None:
        return None
    tf = rec["fp32_flops_per_launch"] / (kern_ms * 1e-3) / 1e12
    return {"achieved": round(tf, 2), "unit": "TFLOP/s", "peak": VALU_PEAK_TFLOPS,
            "frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "peak_without_packed_fp32": VALU_PEAK_UNPACKED_TFLOPS,
            "frac_without_packed_fp32": round(tf / VALU_PEAK_UNPACKED_TFLOPS, 4),
            "fp32_flops_per_launch": rec["fp32_flops_per_launch"],
            "fp32_flops_per_sample": rec["fp32_flops_per_sample"],
            "valu_instr_per_sample": rec["valu_instr_per_sample"]}


WORKLOAD_NOTE = {
    "cfg1": "M=65, N=256, 12288 samples",
    "cfg2": "M=1025, N=4096, 4 calls of 786432 samples",
    "cfg3": "M=8193, N=32768, 50331648 samples",
    "cfg4": "M=16385, N=65536 via H, 251658240 samples",
    "cfg5": "M=257, N=1024, 1024 channels x 65536 samples",
    "n1048576": "M=262145, N=1048576, one call of 170 blocks (tune_n.py --logn 20 20)",
    "n16384": "M=4097, N=16384, one call of 10922 blocks (tune_n.py --logn 14 14)",
    "pfb1024": "channelizer K=1024, D=512, Nh=8192, 2^26 samples per call",
    "pfb128": "channelizer K=128, D=64, Nh=1024, 2^26 samples per call",
}



TABLE_KEYS = ("cfg1", "cfg2", "cfg3", "cfg4", "cfg5")
HEADLINE = "cfg4"   # the largest configuration that fits one GPU


def roofline_kernel(N: int) -> str:
    """Name of the filtering kernel of a plan with N-point blocks, as the
    profiles print it."""
    return (f"ols_fused_kernel<{int(np.log2(N))}, false>" if N <= 8192 else
            "ols_mid_kernel<false>" if N == 16384 else
            "ols_big_kernel<false>" if N == 32768 else
            "ols_pair_kernel<false>" if N == 65536 else "ols_multi_sub_kernel<false>")


def measure(key, fo, torch, *, steps, warmup, timed_ms, warm_ms, cpu_budget, cpu_single_s,
            do_parity, do_cpu, headline=False, args=None):
    """Time one workload: W untimed warm-up steps, then exactly K timed steps
    between two HIP events on the launch stream (K and W sized from a probe
    to about timed_ms and warm_ms when not given).  Returns its record."""
    import workloads as W
    dev = torch.device("cuda:0")
    inp = W.make_inputs(key)
    w = inp.workload
    samples_per_step = w.nchan * w.samples
    step_bytes = samples_per_step * BYTES_PER_SAMPLE
    nsets = max(1, min(64, -(-2 * LLC_BYTES // step_bytes)))
    print(f"# workload {w.key}: {w.description}; {nsets} buffer set(s)", file=sys.stderr,
          flush=True)

    x_host = torch.from_numpy(inp.x)
    xs = [x_host.to(dev) for _ in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    plan = fo.Plan(w.M, w.N, w.nchan)
    if inp.H is not None:
        plan.set_freq_response(inp.H)
    else:
        plan.set_taps(inp.taps)
    s0_dev = torch.from_numpy(inp.s0).to(dev)
    plan.set_state(s0_dev)
    item = 8
    stride = w.samples

    def step(k):
        x, y = xs[k % nsets], ys[k % nsets]
        pos = 0
        for c in w.calls:
            fo.fir_ols_execute(plan.handle, x.data_ptr() + pos * item,
                               y.data_ptr() + pos * item, c, stride, sptr)
            pos += c

    # parity of one step against the oracle (fresh state, before timing)
    parity, ref, base = None, None, None
    if do_cpu:
        base, ref = cpu_baseline(inp, cpu_budget, cpu_single_s)
    if do_parity:
        import oracle
        plan.set_state(s0_dev)
        step(0)
        torch.cuda.synchronize()
        y0 = ys[0].cpu().numpy()
        if ref is not None and ref.shape == y0.shape:
            yref, idx = ref, None
        else:
            idx = W.sample_indices(7, w.samples, 4096)
            yref = oracle.fir_direct_multi(inp.h_ref, inp.x, inp.s0, idx=idx,
                                           threads=len(os.sched_getaffinity(0)))
            y0 = y0[:, idx]
        err = float(np.abs(y0.astype(np.complex128) - yref).max())
        bound = oracle.parity_bound(inp.h_ref, inp.x, inp.s0)
        parity = {"max_abs_err": err, "bound": bound, "ok": err <= bound,
                  "outputs_checked": int(yref.size)}
        del y0, yref
    ref = None

    # size the default warm-up and step counts from a short probe
    probe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step(0)
    probe[0].record(stream)
    for k in range(5):
        step(k)
    probe[1].record(stream)
    torch.cuda.synchronize()
    est_ms = max(probe[0].elapsed_time(probe[1]) / 5, 1e-3)
    if warmup < 0:
        warmup = max(20, int(warm_ms / est_ms))
    if steps <= 0:
        steps = max(20, int(timed_ms / est_ms))
    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()

    ncalls = len(w.calls)
    # timed region: exactly K steps, nothing else on the stream
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(steps):
        step(k)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / steps
    value = samples_per_step / (ms_per_step * 1e-3) / 1e6

    # per-launch duration of the filtering kernel: the HIP events around the
    # timed region (on the launch stream) over the launches in it; a step
    # launches the filtering kernel once per call (N <= 65536) and nothing else
    launches = ncalls if w.N <= 65536 else None
    kern_ms = total_ms / (steps * ncalls)
    kern_bytes = samples_per_step / ncalls * BYTES_PER_SAMPLE
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.key)

    rec = {
        "value": round(value, 1),
        "unit": "Msamples/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "config": {
            "workload": f"{w.key}: {w.description}",
            "M": w.M, "N": w.N, "L": w.L, "nchan": w.nchan,
            "calls_per_step": ncalls, "samples_per_step": samples_per_step,
            "buffer_sets": nsets,
            "hbm_roof_fraction": round(value * 1e6 * BYTES_PER_SAMPLE / (HBM_PEAK_GBPS * 1e9), 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": roofline_kernel(w.N),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_ratio": (round(traffic / kern_bytes, 3) if traffic else None),
            "avg_launch_us": round(kern_ms * 1e3, 3),
            "avg_launch_source": "HIP events around the timed region on the launch stream, "
                                 "divided by the launches in it (includes the gaps between "
                                 "launches)",
            "kernel_launches_per_step": launches,
            "kernel_source_hash": kernel_source_hash(w.key),
            "algorithmic_bytes_per_launch": int(kern_bytes),
        },
        "valu": valu_line(w.key, kern_ms),
        "parity": parity,
        "cpu_baseline": base,
        "wall_s": round(wall, 3),
    }
    if base is not None:
        rec["gpu_over_oracle"] = round(value / base["value"], 1)

    if headline:
        # copy reference: the same bytes through a plain elementwise kernel
        # (one read and one write per element); also the calibration
        # dispatch of the FETCH_SIZE / WRITE_SIZE counter runs
        fx = [x.view(torch.float32).view(-1) for x in xs]
        fy = [y.view(torch.float32).view(-1) for y in ys]
        for r in range(3):
            torch.neg(fx[r % nsets], out=fy[r % nsets])
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        reps = max(5, min(200, int(200.0 / max(est_ms, 1e-3))))
        torch.cuda.synchronize()
        c0.record(stream)
        for r in range(reps):
            torch.neg(fx[r % nsets], out=fy[r % nsets])
        c1.record(stream)
        torch.cuda.synchronize()
        rec["copy_reference_GBps"] = round(
            reps * 2 * fx[0].numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
        del fx, fy
    plan.close()
    if headline and args is not None:
        rec["host_stream"] = (host_stream(args, inp, fo, torch, stream)
                              if args.host_stream else None)
        rec["real_pairs"] = real_pairs(inp, fo, torch, stream, nsets) if args.real else None
    del xs, ys, x_host, s0_dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def table_row(rec):
    """The per-configuration summary kept in the bench line's "configs"."""
    cfg = rec["config"]
    roof = rec["roofline"]
    base = rec.get("cpu_baseline") or {}
    par = rec.get("parity") or {}
    return {"workload": cfg["workload"], "M": cfg["M"], "N": cfg["N"], "nchan": cfg["nchan"],
            "calls_per_step": cfg["calls_per_step"],
            "samples_per_step": cfg["samples_per_step"], "steps": rec["steps"],
            "warmup": rec["warmup"], "ms_per_step": rec["ms_per_step"],
            "Msamples_per_s": rec["value"], "hbm_roof_fraction": cfg["hbm_roof_fraction"],
            "kernel": roof["kernel"], "kernel_frac": roof["frac"],
            "avg_launch_us": roof["avg_launch_us"], "traffic_ratio": roof["traffic_ratio"],
            "valu_tflops": (rec["valu"] or {}).get("achieved"),
            "parity_ok": par.get("ok"), "parity_max_abs_err": par.get("max_abs_err"),
            "parity_bound": par.get("bound"), "outputs_checked": par.get("outputs_checked"),
            "oracle_Msamples_per_s": base.get("value"), "oracle_cores": base.get("cores"),
            "oracle_sample": base.get("sample"),
            "oracle_single_thread_Msamples_per_s": base.get("single_thread_value"),
            "gpu_over_oracle": rec.get("gpu_over_oracle")}


def main():
    args = parse()
    global PROFILES_DIR
    if args.profiles_dir:
        PROFILES_DIR = args.profiles_dir
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_valu:
        summarize_valu(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import order_fir_filtering_amd as fo
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    fo.load_library()

    if args.workload in W.PFB_WORKLOADS:
        # the channelizer alone: its own line, same contract fields
        args.channelizer = args.workload
        wall0 = time.perf_counter()
        ch = channelizer(args, fo, torch, torch.cuda.current_stream())
        line = {"metric": ch.pop("metric"), "value": ch.pop("value"), "unit": ch.pop("unit"),
                "n_gpus": 1, "steps": ch.pop("steps"), "warmup": 5,
                "ms_per_step": ch.pop("ms_per_call"), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                "config": {"workload": ch.pop("workload"), "K": ch.pop("K"), "D": ch.pop("D"),
                           "Nh": ch.pop("Nh"), "samples_per_step": ch.pop("samples_per_call"),
                           "outputs_per_step": ch.pop("outputs_per_call")},
                "roofline": ch.pop("roofline"), "parity": ch.pop("parity"),
                "cpu_baseline": ch.pop("cpu_baseline", None),
                "wall_s": round(time.perf_counter() - wall0, 3)}
        print(json.dumps(line), flush=True)
        return

    wall0 = time.perf_counter()
    # every other configuration first (each with its own warm-up, timing,
    # sampled parity and a short oracle baseline); this also brings the
    # clocks up before the headline is timed
    table = {}
    if not args.no_table:
        for key in TABLE_KEYS:
            if key == args.workload:
                continue
            rec = measure(key, fo, torch, steps=0, warmup=-1, timed_ms=300.0, warm_ms=200.0,
                          cpu_budget=3.0, cpu_single_s=0.5, do_parity=not args.no_parity,
                          do_cpu=not args.no_cpu_baseline)
            table[key] = table_row(rec)
            print(f"# {key}: {rec['value']:.0f} Msamples/s, kernel {rec['roofline']['frac']:.3f} "
                  f"of the HBM roof", file=sys.stderr, flush=True)

    head = measure(args.workload, fo, torch, steps=args.steps, warmup=args.warmup,
                   timed_ms=1000.0, warm_ms=1000.0, cpu_budget=15.0, cpu_single_s=2.0,
                   do_parity=not args.no_parity, do_cpu=not args.no_cpu_baseline,
                   headline=True, args=args)
    if not args.no_table:
        table[args.workload] = table_row(head)
        table = {k: table[k] for k in sorted(table)}
    chan = channelizer(args, fo, torch, torch.cuda.current_stream()) if args.channelizer else None
    out = {
        "metric": "filtered output Msamples/s (complex fp32) and % of HBM roof, per (M,N)",
        "value": head["value"],
        "unit": "Msamples/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "valu": head["valu"],
        "copy_reference_GBps": head.get("copy_reference_GBps"),
        "parity": head["parity"],
        "cpu_baseline": head["cpu_baseline"],
        "gpu_over_oracle": head.get("gpu_over_oracle"),
        "configs": table or None,
        "host_stream": head.get("host_stream"),
        "real_pairs": head.get("real_pairs"),
        "channelizer": chan,
        "page_context": "the method page's abstract reports a typical speedup above 100x over "
                        "a single-threaded CPU overlap-save (hardware not stated); context only",
        "wall_s": head["wall_s"],
        "bench_wall_s": round(time.perf_counter() - wall0, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
