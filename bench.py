#!/usr/bin/env python3
"""Benchmark of the MoE dispatch + combine hot path on one MI355X.

One step = one moe_dispatch (route count, scan, slots, fused fp8 pack and
scatter) followed by one moe_combine (weighted f32 gather-reduce, bf16 out,
out_weights) over the skewed_fp8 workload: T=8192 tokens, H=7168, E=256
experts, K=8 distinct Zipf(1.2) picks, bf16 x, fp8 e4m3 payload with f32
scales per 128 elements, bf16 expert outputs.  The expert step (fp8
dequantize, the identity expert) runs once per buffer set before the timed
region; dispatch is deterministic, so its output is the same on every step.

Inputs sit in HBM before timing starts.  Several buffer sets rotate so the
256 MB Infinity Cache cannot serve a step's inputs from the previous step.

Prints ONE JSON line on stdout.  Other lines go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs/call and achieved HBM GB/s (% of peak), T=8192 H=7168 K=8"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(T, H, K, E, N_rows, fp8=True, y_bytes=2, out_bytes=2, y_fp8=False, fp4=False):
    """Bytes the method must move per call (metadata once, rows once).  y_fp8:
    the combine reads the quantized expert outputs (one f32 scale per 128
    elements); fp4: the payload is e2m1, two codes per byte."""
    idx = T * K * 4
    tok_map = T * K * 8
    w = T * K * 4
    x = T * H * 2
    qrow = H // 2 if fp4 else H
    if fp8:
        rows_w = N_rows * qrow + N_rows * (H // 128) * 4
    else:
        rows_w = N_rows * H * 2
    meta_d = idx + tok_map + N_rows * 4 + E * 4 * 2   # idx in, tok_map/packed_src/cnt/off out
    disp = x + rows_w + meta_d
    comb_rows = N_rows * qrow + N_rows * (H // 128) * 4 if y_fp8 else N_rows * H * y_bytes
    comb = comb_rows + T * H * out_bytes + tok_map + w + T * 4
    return disp, comb


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


COMBINE_SOURCES = ["combine_moe_route_count_amd/csrc/combine.hip",
                   "combine_moe_route_count_amd/csrc/device_common.hpp",
                   "combine_moe_route_count_amd/csrc/geometry.cpp"]


def stored_profile(kernel_hash):
    """The committed rocprofv3 summary of the combine kernel (HBM bytes per launch
    from the counters, average duration from the kernel trace), or {} when it is
    missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "combine_skewed_fp8_pmc.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        d = json.load(f)
    if d.get("combine_source_hash") != kernel_hash:
        return {}
    return d


COPY_BYTES = 1 << 30   # calibration copy: 1 GiB read + 1 GiB written per launch


def calibrate_copy(steps):
    """The library's 16-byte streaming copy of known size, profiled with the same
    counters as the kernels so their KiB readings can be scaled to bytes."""
    import torch
    import combine_moe_route_count_amd as moe
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(steps):
        moe.copy16(a, b)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {COPY_BYTES} bytes x {steps} done")


# The headline combine (bf16 y, bf16 out, K <= 8) as its name starts in the trace.
HEADLINE_COMBINE = "combine_kernel<false, false, 8>"


def _pmc_rows(path, kernel_prefix):
    import csv
    vals = []
    for r in csv.DictReader(open(path)):
        if _short_kernel(r["Kernel_Name"]).startswith(kernel_prefix):
            vals.append(float(r["Counter_Value"]))
    return vals


def pmc_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, out_json, trace_avg_us=None):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the headline combine
    kernel, scaled by what the same counters read for the 1 GiB calibration
    copy; with the kernel trace's average duration of that kernel when given."""
    f = _pmc_rows(fetch_csv, HEADLINE_COMBINE)
    wv = _pmc_rows(write_csv, HEADLINE_COMBINE)
    cf = _pmc_rows(cal_fetch_csv, "copy16_kernel")
    cw = _pmc_rows(cal_write_csv, "copy16_kernel")
    cf_avg = statistics.mean(x for x in cf if x > 0)
    cw_avg = statistics.mean(x for x in cw if x > 0)
    fetch_scale = COPY_BYTES / cf_avg     # bytes per counter unit
    write_scale = COPY_BYTES / cw_avg
    f_avg, w_avg = statistics.mean(f), statistics.mean(wv)
    d = {"kernel": "combine_kernel", "workload": "skewed_fp8 T=8192 H=7168 E=256 K=8",
         "fetch_size_avg": f_avg, "write_size_avg": w_avg, "dispatches": [len(f), len(wv)],
         "calibration_copy_bytes": COPY_BYTES, "calibration_fetch_size": cf_avg,
         "calibration_write_size": cw_avg, "fetch_bytes_per_unit": fetch_scale,
         "write_bytes_per_unit": write_scale,
         "fetch_bytes_per_launch": f_avg * fetch_scale, "write_bytes_per_launch": w_avg * write_scale,
         "traffic_bytes_per_launch": f_avg * fetch_scale + w_avg * write_scale,
         "trace_avg_us": trace_avg_us,
         "combine_source_hash": source_hash(COMBINE_SOURCES)}
    with open(out_json, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d, indent=1))


# rocprofv3 runs behind the committed summaries under profiles/ (run with -d DIR,
# then `python bench.py --profile-text DIR profiles`).  The kernel trace covers a
# default bench run without the CPU leg; the counter runs, one per workload so
# that kernels shared by several workloads are not mixed, read FETCH_SIZE and
# WRITE_SIZE in runs of their own, and the library's 1 GiB copy calibrates them.
PROFILE_WORKLOADS = {
    "skewed_fp8": "--steps 5 --warmup 2 --no-cpu --no-graph --no-latency --secondary none --no-dedup",
    "uniform_bf16": "--workload uniform_bf16 --steps 5 --warmup 2 --no-cpu --no-graph --no-latency "
                    "--secondary none --no-dedup",
    "dedup": "--only-dedup --steps 5 --warmup 2",
    "prefill": "--latency-configs --latency-names prefill --latency-reps 5",
}
PROFILE_RUNS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace -o bench -- "
             "python bench.py --steps 10 --warmup 5 --no-cpu --no-latency",
    # the headline pair alone: the combine kernel also serves the uniform_bf16
    # line, so the full trace's average mixes two workloads
    "trace_headline": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/trace_headline "
                      "-o bench -- python bench.py --steps 30 --warmup 20 --no-cpu --no-latency "
                      "--no-graph --no-fp --secondary none --no-dedup",
    "cal_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}/cal_FETCH_SIZE -o copy -- "
                      "python bench.py --calibrate-copy --steps 3",
    "cal_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}/cal_WRITE_SIZE -o copy -- "
                      "python bench.py --calibrate-copy --steps 3",
}
for _w, _a in PROFILE_WORKLOADS.items():
    for _c in ("FETCH_SIZE", "WRITE_SIZE"):
        PROFILE_RUNS[f"{_w}_{_c}"] = (f"rocprofv3 --pmc {_c} --output-format csv -d {{d}}/{_w}_{_c} "
                                      f"-o bench -- python bench.py {_a}")


def _short_kernel(name):
    import re
    name = re.sub(r"^void ", "", name)
    name = name.replace("moe::(anonymous namespace)::", "").replace("moe::", "")
    name = re.sub(r"\((\w+)\)(\d+)", r"\1=\2", name)   # enum template arguments
    if not name.startswith("at::"):
        name = re.sub(r"\(.*$", "", name)
    return name[:90]


LATENCY_PROFILE_RUN = ("rocprofv3 --kernel-trace --stats --output-format csv -d {d}/latency -o lat -- "
                       "python bench.py --latency-configs")


def latency_profile_text(prof_dir, out_dir):
    """Text summary of the kernel trace of the --latency-configs run (tiny, decode
    and prefill; eager then graph-replayed pairs)."""
    import csv
    cmd = LATENCY_PROFILE_RUN.format(d=prof_dir)
    stats = list(csv.DictReader(open(os.path.join(prof_dir, "latency", "lat_kernel_stats.csv"))))
    out = ["# Kernel trace: the tiny (T=64 H=256 E=8 K=2), decode (T=32 H=6144 E=128 K=8) and",
           "# prefill (T=4096 H=7168 E=256 K=8, padded) configurations, MI355X",
           f"# command: {cmd}",
           "# (bench.py --latency-configs: per configuration 1 setup dispatch, 70 eager pairs and",
           "#  70 graph replays, a 2e6-cycle sleep kernel ahead of each pair)",
           f"# summary: python bench.py --latency-profile-text {prof_dir} profiles",
           "# kernel | calls | avg us | min us | max us | % of GPU time", ""]
    for r in stats:
        out.append(f"{_short_kernel(r['Name']):70s} {int(r['Calls']):5d} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                   f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    with open(os.path.join(out_dir, "latency_configs_kernel_trace.txt"), "w") as fh:
        fh.write("\n".join(out) + "\n")


def dedup_rows(W):
    """Recv rows (distinct (token, rank) pairs) and packed rows of the dedup
    workload, from its routing alone."""
    import numpy as np
    d = W.make_inputs("dedup")
    er = d["E"] // d["R"]
    idx = d["idx"]
    valid = (idx >= 0) & (idx < d["E"])
    ranks = np.where(valid, idx // er, -1)
    n_recv = sum(len(set(r[r >= 0].tolist())) for r in ranks)
    return d, n_recv, int(valid.sum())


def kernel_algorithmic_bytes(W):
    """Algorithmic bytes per launch (or per call, for groups of kernels) of the
    kernels the counter summaries compare against, by workload."""
    out = {}
    db, cb = algorithmic_bytes(8192, 7168, 8, 256, 8192 * 8, fp8=True)
    out["skewed_fp8"] = {("route_fused_kernel<ExpertKeys>", "scatter_fp8_kernel<8, 2, false, false>"): db,
                         (HEADLINE_COMBINE,): cb}
    db, cb = algorithmic_bytes(8192, 7168, 8, 256, 8192 * 8, fp8=False)
    out["uniform_bf16"] = {("route_fused_kernel<ExpertKeys>", "scatter_copy_kernel<8, 4, false, false>"): db,
                           (HEADLINE_COMBINE,): cb}
    db, cb = algorithmic_bytes(4096, 7168, 8, 256, 4096 * 8, fp8=False)
    out["prefill"] = {("route_fused_kernel<ExpertKeys>", "scatter_copy_kernel<8, 4, false, false>"): db,
                      (HEADLINE_COMBINE,): cb}
    d, n_recv, n_rows = dedup_rows(W)
    T, H, K, R = d["T"], d["H"], d["K"], d["R"]
    row = H * 4
    meta_d = T * K * 4 + T * K * 8 + n_rows * 4 + n_recv * 4 + T * R * 4
    comb_fused = n_rows * row + T * row + T * K * 16 + T * R * 4 + T * 4
    out["dedup"] = {("route_fused_kernel<RankKeys>", "recv_copy_kernel<8, 4>",
                     "route_fused_kernel<SurvivorKeys>", "expand_kernel<8, 4>"):
                    T * row + 2 * n_recv * row + n_rows * row + meta_d,
                    ("recv_copy_kernel<8, 4>",): T * row + n_recv * row,
                    ("expand_kernel<8, 4>",): n_recv * row + n_rows * row,
                    ("dedup_combine_kernel<true, true, 6, 0>",): comb_fused,
                    ("dedup_combine_kernel<true, true, 6, 1>", "dedup_sum_kernel<true, 6>"):
                    comb_fused + 2 * n_recv * row}
    return out


def profile_text(prof_dir, out_dir):
    """Text summaries of the rocprofv3 runs in PROFILE_RUNS (run with -d prof_dir):
    per-kernel trace statistics, HBM bytes per dispatch from FETCH_SIZE /
    WRITE_SIZE scaled by the 1 GiB calibration copy (per workload, against the
    algorithmic bytes), and the headline combine's counter / trace JSON."""
    import collections
    import csv
    import workloads as W
    cmd = {k: v.format(d=prof_dir) for k, v in PROFILE_RUNS.items()}
    stats = list(csv.DictReader(open(os.path.join(prof_dir, "trace", "bench_kernel_stats.csv"))))
    out = ["# Kernel trace of a default bench.py run without the CPU leg, MI355X:",
           "#  the headline skewed_fp8 pair (T=8192 H=7168 E=256 K=8, Zipf 1.2, fp8 payload):",
           "#  3 setup dispatches + dequants, 5 warmup, 2x10 timed, 3 + 5 + 10 graph-replayed pairs",
           "#  and as many split dispatch / combine replays; the uniform_bf16 line (same shape,",
           "#  uniform routing, bf16 payload) the same way; the fp8-input combine pair, the fp4",
           "#  payload pair, the dispatch variants (replay, pre-quantized); the dedup line",
           "#  (T=16384 H=4096 E=64 K=6 R=8 f32); the 1 GiB 16-byte copy ceiling",
           f"# command: {cmd['trace']}",
           f"# summary: python bench.py --profile-text {prof_dir} profiles",
           "# kernel | calls | avg us | min us | max us | % of GPU time", ""]
    for r in stats:
        k = _short_kernel(r["Name"])
        out.append(f"{k:70s} {int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):6.2f}")
    with open(os.path.join(out_dir, "skewed_fp8_kernel_trace.txt"), "w") as fh:
        fh.write("\n".join(out) + "\n")
    # the headline pair alone (the source of the combine's trace average)
    hstats = list(csv.DictReader(open(os.path.join(prof_dir, "trace_headline",
                                                   "bench_kernel_stats.csv"))))
    head_avg = {}
    hout = ["# Kernel trace of the headline skewed_fp8 pair alone (T=8192 H=7168 E=256 K=8, Zipf 1.2,",
            "#  fp8 payload, bf16 expert outputs), MI355X: 3 setup dispatches + dequants, 20 warmup,",
            "#  30 back-to-back and 2x30 event-timed pairs",
            f"# command: {cmd['trace_headline']}",
            f"# summary: python bench.py --profile-text {prof_dir} profiles",
            "# kernel | calls | avg us | min us | max us | % of GPU time", ""]
    for r in hstats:
        k = _short_kernel(r["Name"])
        head_avg.setdefault(k, float(r["AverageNs"]) / 1e3)
        hout.append(f"{k:70s} {int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:9.2f} "
                    f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                    f"{float(r['Percentage']):6.2f}")
    with open(os.path.join(out_dir, "skewed_fp8_headline_kernel_trace.txt"), "w") as fh:
        fh.write("\n".join(hout) + "\n")

    def per_kernel(sub, name):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(prof_dir, sub, name))):
            d[_short_kernel(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return d

    cf = statistics.mean(x for x in per_kernel("cal_FETCH_SIZE", "copy_counter_collection.csv")
                         ["copy16_kernel"] if x > 0)
    cw = statistics.mean(x for x in per_kernel("cal_WRITE_SIZE", "copy_counter_collection.csv")
                         ["copy16_kernel"] if x > 0)
    fs, wsc = COPY_BYTES / cf, COPY_BYTES / cw
    alg = kernel_algorithmic_bytes(W)
    lines = ["# HBM traffic per kernel dispatch from rocprofv3 counters, MI355X, one counter run per",
             "# workload and counter (kernels shared by several workloads are not mixed)", "# commands:"]
    lines += [f"#   {cmd[k]}" for k in PROFILE_RUNS if not k.startswith("trace")]
    lines += [f"#   python bench.py --profile-text {prof_dir} profiles",
              f"# calibration: the library's 16-byte copy of 1 GiB reads FETCH_SIZE {cf:.0f} and "
              f"WRITE_SIZE {cw:.0f};",
              f"#   bytes per counter unit: fetch {fs:.1f}, write {wsc:.1f}",
              "# kernel | dispatches | fetch MB | write MB (averages per dispatch, scaled)", ""]
    headline = None
    for wl in PROFILE_WORKLOADS:
        fetch = per_kernel(f"{wl}_FETCH_SIZE", "bench_counter_collection.csv")
        write = per_kernel(f"{wl}_WRITE_SIZE", "bench_counter_collection.csv")
        lines.append(f"## {wl}: python bench.py {PROFILE_WORKLOADS[wl]}")
        tot = {}
        for k in fetch:
            if k not in write or not k or k.startswith("at::") or k.startswith("__amd"):
                continue
            fb = statistics.mean(fetch[k]) * fs
            wb = statistics.mean(write[k]) * wsc
            tot[k] = fb + wb
            lines.append(f"{k:70s} {len(fetch[k]):4d} {fb / 1e6:10.2f} {wb / 1e6:10.2f}")
        for group, b in alg.get(wl, {}).items():
            if all(k in tot for k in group):
                t = sum(tot[k] for k in group)
                lines.append(f"  {' + '.join(group)}: algorithmic {b} B, counters {t:.0f} B "
                             f"({t / b:.4f}x)")
                if wl == "skewed_fp8" and group == (HEADLINE_COMBINE,):
                    headline = (fetch[HEADLINE_COMBINE], write[HEADLINE_COMBINE])
        lines.append("")
    with open(os.path.join(out_dir, "hbm_counters.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    pmc_summary(os.path.join(prof_dir, "skewed_fp8_FETCH_SIZE", "bench_counter_collection.csv"),
                os.path.join(prof_dir, "skewed_fp8_WRITE_SIZE", "bench_counter_collection.csv"),
                os.path.join(prof_dir, "cal_FETCH_SIZE", "copy_counter_collection.csv"),
                os.path.join(prof_dir, "cal_WRITE_SIZE", "copy_counter_collection.csv"),
                os.path.join(out_dir, "combine_skewed_fp8_pmc.json"),
                trace_avg_us=head_avg.get(HEADLINE_COMBINE))


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family / model /
    stepping, and the clock it reports."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                info.setdefault(k.strip(), v.strip())
            if not line.strip() and info:
                break
    except OSError:
        return None
    return (f"{info.get('model name', '?')} (family {info.get('cpu family', '?')}, model "
            f"{info.get('model', '?')}, stepping {info.get('stepping', '?')}, "
            f"{info.get('cpu MHz', '?')} MHz)")


def _cpu_topology():
    """(logical CPUs in this process's affinity mask, distinct physical cores among them)."""
    cpus = sorted(os.sched_getaffinity(0))
    cores = set()
    for c in cpus:
        base = f"/sys/devices/system/cpu/cpu{c}/topology/"
        try:
            cores.add((open(base + "physical_package_id").read().strip(),
                       open(base + "core_id").read().strip()))
        except OSError:
            cores.add(("cpu", str(c)))
    return len(cpus), len(cores)


def cpu_child(name, reps, threads):
    """Runs in a child process started by cpu_baseline, with its OpenMP binding
    environment set: the oracle as it stands on the full workload with a team
    of `threads` (omp_set_num_threads), one warmup call then `reps` timed calls
    of dispatch and combine (the expert step, the fp8 dequantize, is untimed).
    Prints one JSON line, with the binding the OpenMP runtime reports."""
    import ctypes
    import oracle
    import workloads as W
    oracle.set_threads(threads)
    gomp = ctypes.CDLL("libgomp.so.1")
    bind = ["false", "true", "primary", "close", "spread"][gomp.omp_get_proc_bind()]
    places = gomp.omp_get_num_places()
    d = W.make_inputs(name)
    E = d["E"]
    fp8 = d["packed_dtype"] == "fp8"
    disp, comb = [], []
    for rep in range(1 + reps):
        t0 = time.perf_counter()
        ref = oracle.dispatch(d["x"], "bf16", d["idx"], E, packed_dt="fp8" if fp8 else None)
        t1 = time.perf_counter()
        y = oracle.fp8_dequant(ref["packed"], ref["scales"]) if fp8 else ref["packed"]
        t2 = time.perf_counter()
        oracle.combine(y, "bf16", ref["tok_map"], d["w"], "bf16")
        t3 = time.perf_counter()
        if rep > 0:
            disp.append((t1 - t0) * 1e6)
            comb.append((t3 - t2) * 1e6)
        del ref, y
    pair = [a + b for a, b in zip(disp, comb)]
    print(json.dumps({"threads": oracle.get_threads(), "proc_bind": bind, "places": places,
                      "dispatch_us": statistics.median(disp),
                      "combine_us": statistics.median(comb), "pair_us": statistics.median(pair),
                      "pair_us_all": pair}), flush=True)


def cpu_baseline(name, bytes_full, reps=5):
    """The oracle, as it stands, timed on this host on the full workload: one
    thread per physical core of the affinity mask (OMP_PLACES=cores,
    OMP_PROC_BIND=close: never two SMT siblings), capped by the host's CPU share
    when OMP_NUM_THREADS gives one, and again on one thread; each 1 warmup +
    median of `reps`.  Each run is a child process, so its OpenMP runtime
    starts with that environment."""
    import subprocess
    n_cpus, n_phys = _cpu_topology()
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(n_phys, int(share)) if share.isdigit() and int(share) > 0 else n_phys

    def run(nthreads):
        env = dict(os.environ, OMP_PLACES="cores", OMP_PROC_BIND="close")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child", name,
                            str(reps), str(nthreads)], env=env, capture_output=True, text=True,
                           timeout=900)
        if r.returncode != 0:
            raise RuntimeError(f"cpu baseline child failed:\n{r.stderr[-2000:]}")
        return json.loads(r.stdout.strip().splitlines()[-1])

    a = run(threads)
    log(f"[bench] cpu oracle on {a['threads']} threads: {a['pair_us']:.0f} us/call")
    one = run(1)
    log(f"[bench] cpu oracle on {one['threads']} thread: {one['pair_us']:.0f} us/call")
    assert one["threads"] == 1 and a["threads"] == threads, (a["threads"], one["threads"])
    gb = lambda us: round(bytes_full / (us * 1e-6) / 1e9, 2)
    return {"value": round(a["pair_us"], 1), "unit": "us/call", "cores": a["threads"],
            "kind": "oracle",
            "sample": f"the full {name} workload (every token), dispatch + combine per call; "
                      f"1 warmup + median of {reps} calls; expert step (fp8 dequantize) untimed",
            "dispatch_us": round(a["dispatch_us"], 1), "combine_us": round(a["combine_us"], 1),
            "gbps": gb(a["pair_us"]),
            "single_thread_value": round(one["pair_us"], 1),
            "single_thread_dispatch_us": round(one["dispatch_us"], 1),
            "single_thread_combine_us": round(one["combine_us"], 1),
            "single_thread_gbps": gb(one["pair_us"]),
            "omp": f"OMP_PLACES=cores OMP_PROC_BIND=close (runtime reports proc_bind "
                   f"{a['proc_bind']}, {a['places']} places)",
            "affinity_cpus": n_cpus, "physical_cores_in_affinity": n_phys,
            "host_cpu_share": int(share) if share.isdigit() else None,
            "cpu_model": _cpu_model()}


def measure(moe, W, name, args, dev, graphs=True, y_fp8=False, fp4=False):
    """Time dispatch+combine pairs of one workload; returns medians and spreads.

    Pass 1 (the headline): HIP events on the launch stream around each
    dispatch+combine pair, none between the two calls.  y_fp8: the combine takes
    the fp8 packed rows and scales themselves (moe_combine_fp8, identity expert);
    fp4 (with y_fp8): an e2m1 payload end to end (moe_combine_fp4).  Pass 2 (breakdown): a
    marker between dispatch and combine as well.  Pass 3: each pair replayed
    from a captured HIP graph, its outputs checked against the eager ones."""
    import numpy as np
    import torch

    d = W.make_inputs(name)
    T, H, E, K = d["T"], d["H"], d["E"], d["K"]
    fp8 = d["packed_dtype"] == "fp8"
    assert d["x_dtype"] == "bf16" and (fp8 or not y_fp8)
    log(f"[bench] workload {name}: T={T} H={H} E={E} K={K} fp8={fp8} y_fp8={y_fp8} sets={args.sets}")
    x0 = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(d["idx"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    ws = moe.workspace(T, K, E, 0, dev)
    sets = []
    for s_ in range(args.sets):
        x = x0.clone()
        o = moe.dispatch(x, idx, E, fp8=fp8 and not fp4, ws=ws, fp4=fp4)
        if y_fp8:
            y = None
        else:
            y = moe.fp8_dequant(o.packed, o.scales) if fp8 else o.packed.clone()
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ow = torch.empty(T, dtype=torch.float32, device=dev)
        sets.append(dict(x=x, o=o, y=y, out=out, ow=ow))
    del x0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def dispatch_call(st):
        moe.dispatch(st["x"], idx, E, fp8=fp8 and not fp4, out=st["o"], ws=ws, fp4=fp4)

    def combine_call(st):
        if y_fp8:
            qc = moe.combine_fp4 if fp4 else moe.combine_fp8
            qc(st["o"].packed, st["o"].scales, st["o"].tok_map, w, out=st["out"], out_weights=st["ow"])
        else:
            moe.combine(st["y"], st["o"].tok_map, w, out=st["out"], out_weights=st["ow"])

    def step(i, events=None):
        st = sets[i % len(sets)]
        if events is not None:
            events[0].record(stream)
        dispatch_call(st)
        if events is not None and len(events) == 3:
            events[1].record(stream)
        combine_call(st)
        if events is not None:
            events[-1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] {name}: warmup {args.warmup} done")

    # wall clock over exactly `steps` back-to-back steps, no event markers
    # between them (each marker leaves the GPU idle for several microseconds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps

    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    log(f"[bench] {name}: timed {args.steps} steps done")
    pair_us = [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in range(n_ev)]

    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for i in range(args.steps):
        step(i, evb[i])
    torch.cuda.synchronize()
    disp_us = [evb[i][0].elapsed_time(evb[i][1]) * 1e3 for i in range(n_ev)]
    comb_us = [evb[i][1].elapsed_time(evb[i][2]) * 1e3 for i in range(n_ev)]

    # correctness spot check (identity expert telescopes: weights sum to 1)
    st = sets[(args.steps - 1) % len(sets)]
    assert int(st["o"].stats[1].item()) == 0 and int(st["o"].stats[0].item()) == 0
    ow_err = float((st["ow"] - 1.0).abs().max().item())
    assert ow_err < 1e-5, ow_err

    graph_us = None
    if graphs:
        eager_out = [st_["out"].clone() for st_ in sets]
        cs = torch.cuda.Stream(dev)
        cs.wait_stream(stream)
        gs = []
        with torch.cuda.stream(cs):
            for i in range(len(sets)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    step(i)
                gs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            gs[i % len(gs)].replay()
        evg = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
        for i in range(args.steps):
            evg[i][0].record(stream)
            gs[i % len(gs)].replay()
            evg[i][1].record(stream)
        torch.cuda.synchronize()
        graph_us = [evg[i][0].elapsed_time(evg[i][1]) * 1e3 for i in range(n_ev)]
        for st_, ref in zip(sets, eager_out):
            assert torch.equal(st_["out"].view(torch.int16), ref.view(torch.int16)), \
                "graph replay output differs from the eager output"
        # breakdown in graph mode: dispatch and combine captured as graphs of their own
        gd, gc = [], []
        with torch.cuda.stream(cs):
            for st_ in sets:
                for fn, lst in ((dispatch_call, gd), (combine_call, gc)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cs):
                        fn(st_)
                    lst.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            gd[i % len(gd)].replay()
            gc[i % len(gc)].replay()
        evh = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
        for i in range(args.steps):
            evh[i][0].record(stream)
            gd[i % len(gd)].replay()
            evh[i][1].record(stream)
            gc[i % len(gc)].replay()
            evh[i][2].record(stream)
        torch.cuda.synchronize()
        graph_disp_us = [evh[i][0].elapsed_time(evh[i][1]) * 1e3 for i in range(n_ev)]
        graph_comb_us = [evh[i][1].elapsed_time(evh[i][2]) * 1e3 for i in range(n_ev)]
        for st_, ref in zip(sets, eager_out):
            assert torch.equal(st_["out"].view(torch.int16), ref.view(torch.int16)), \
                "split graph replay output differs from the eager output"
        # one graph holding a step on every buffer set: each launch of a graph
        # leaves the GPU idle for several microseconds before its first kernel
        # (none between its nodes), which a graph of several steps shares out
        for st_ in sets:
            st_["out"].zero_()
        with torch.cuda.stream(cs):
            gm = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gm, stream=cs):
                for i in range(len(sets)):
                    step(i)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // len(sets))):
            gm.replay()
        n_m = max(2, args.steps // len(sets))
        evm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_m)]
        for i in range(n_m):
            evm[i][0].record(stream)
            gm.replay()
            evm[i][1].record(stream)
        torch.cuda.synchronize()
        graph_multi_us = [e[0].elapsed_time(e[1]) * 1e3 / len(sets) for e in evm]
        for st_, ref in zip(sets, eager_out):
            assert torch.equal(st_["out"].view(torch.int16), ref.view(torch.int16)), \
                "multi-step graph replay output differs from the eager output"
        del gs, gd, gc, gm
        log(f"[bench] {name}: graph replays done, outputs equal to eager; pair per graph "
            f"{statistics.median(graph_us[1:]):.1f} us, {len(sets)} pairs per graph "
            f"{statistics.median(graph_multi_us[1:]):.1f} us per pair")

    # drop the first timed round (start transient)
    tail = lambda v: v[1:] if len(v) > 2 else v
    disp_b, comb_b = algorithmic_bytes(T, H, K, E, T * K, fp8=fp8, y_fp8=y_fp8, fp4=fp4)
    r = dict(name=name, T=T, H=H, E=E, K=K, fp8=fp8, routing=d["workload"].routing,
             pair_us=statistics.median(tail(pair_us)), pair_us_min=min(tail(pair_us)),
             pair_us_std=statistics.pstdev(tail(pair_us)),
             dispatch_us=statistics.median(tail(disp_us)), combine_us=statistics.median(tail(comb_us)),
             combine_us_mean=statistics.mean(tail(comb_us)), wall_ms=wall_ms,
             disp_b=disp_b, comb_b=comb_b)
    def spread(v):
        v = tail(v)
        return {"median": round(statistics.median(v), 2), "min": round(min(v), 2),
                "std": round(statistics.pstdev(v), 2)}

    r["timing"] = {"eager": {"pair": spread(pair_us), "dispatch": spread(disp_us),
                             "combine": spread(comb_us)}}
    if graph_us is not None:
        r.update(graph_pair_us=statistics.median(tail(graph_us)), graph_pair_us_min=min(tail(graph_us)),
                 graph_pair_us_std=statistics.pstdev(tail(graph_us)))
        r["timing"]["graph"] = {"pair": spread(graph_us), "dispatch": spread(graph_disp_us),
                                "combine": spread(graph_comb_us)}
        r["timing"]["graph_multi_step"] = {"steps_per_graph": len(sets),
                                           "pair": spread(graph_multi_us)}
        r["graph_multi_pair_us"] = statistics.median(tail(graph_multi_us))
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return r


def dispatch_variants(moe, W, name, args, dev):
    """The dispatch forms around the headline one, on the same fp8 workload:
    replay along a cached tok_map (no routing), the pre-quantized dispatch (fp8
    codes + scale rows forwarded, with routing) and its replay.  Median us of
    args.steps timed calls after args.warmup, 3 rotating buffer sets."""
    import numpy as np
    import torch
    d = W.make_inputs(name)
    T, H, E, K = d["T"], d["H"], d["E"], d["K"]
    stream = torch.cuda.current_stream(dev)
    idx = torch.from_numpy(d["idx"]).to(dev)
    x0 = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    ws = moe.workspace(T, K, E, 0, dev)
    sets = []
    for _ in range(args.sets):
        x = x0.clone()
        o = moe.dispatch(x, idx, E, fp8=True, ws=ws)
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)     # the token rows, pre-quantized
        xs = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
        moe.dispatch_replay(x, torch.arange(T, dtype=torch.int64, device=dev).view(T, 1), xq, scales=xs)
        sets.append(dict(x=x, o=o, xq=xq, xs=xs))
    torch.cuda.synchronize()

    def timeit(fn):
        for i in range(args.warmup):
            fn(sets[i % len(sets)])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(stream)
            fn(sets[i % len(sets)])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
        return statistics.median(us[1:] if len(us) > 2 else us)

    rows = T * K
    meta = T * K * 8 + rows * 4 + E * 8
    b_rep = T * H * 2 + rows * H + rows * (H // 128) * 4 + T * K * 8
    b_pq = T * H + T * (H // 128) * 4 + rows * H + rows * (H // 128) * 4 + T * K * 4 + meta
    b_pqr = T * H + T * (H // 128) * 4 + rows * H + rows * (H // 128) * 4 + T * K * 8
    r_rep = timeit(lambda st: moe.dispatch_replay(st["x"], st["o"].tok_map, st["o"].packed,
                                                  scales=st["o"].scales))
    r_pq = timeit(lambda st: moe.dispatch_prequant(st["xq"], st["xs"], idx, E, out=st["o"], ws=ws))
    r_pqr = timeit(lambda st: moe.dispatch_replay(st["xq"], st["o"].tok_map, st["o"].packed,
                                                  scales=st["o"].scales, x_scales=st["xs"]))
    # the replays and the pre-quantized dispatch reproduce the routed fp8 dispatch
    st = sets[0]
    ref = moe.dispatch(st["x"], idx, E, fp8=True, ws=ws)
    pq = moe.dispatch_prequant(st["xq"], st["xs"], idx, E, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(pq.packed, ref.packed) and torch.equal(pq.tok_map, ref.tok_map)
    del sets
    torch.cuda.empty_cache()
    gb = lambda b, us: round(b / (us * 1e-6) / 1e9, 1)
    res = {"workload": name,
           "replay_fp8_pack": {"us": round(r_rep, 2), "bytes": b_rep, "gbps": gb(b_rep, r_rep)},
           "prequant_dispatch": {"us": round(r_pq, 2), "bytes": b_pq, "gbps": gb(b_pq, r_pq)},
           "prequant_replay": {"us": round(r_pqr, 2), "bytes": b_pqr, "gbps": gb(b_pqr, r_pqr)}}
    log(f"[bench] dispatch variants: replay+fp8 pack {r_rep:.1f} us, pre-quantized {r_pq:.1f} us, "
        f"pre-quantized replay {r_pqr:.1f} us")
    return res


def dedup_line(moe, W, args, dev, name="dedup"):
    """The virtual-rank dedup path on its workload (T=16384 H=4096 E=64 K=6 R=8,
    f32): moe_dedup_dispatch (one recv row per unique (token, rank), then the
    local expansion) and the dedup combine, fused (per-rank partials kept in
    registers) and two-stage (partials written to and read back from HBM, the
    form whose partial rows would cross the links when sharded).  The packed
    rows serve as the expert outputs (identity expert, copied once per set)."""
    import numpy as np
    import torch
    d = W.make_inputs(name)
    T, H, E, K, R = d["T"], d["H"], d["E"], d["K"], d["R"]
    stream = torch.cuda.current_stream(dev)
    idx = torch.from_numpy(d["idx"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    x0 = torch.from_numpy(d["x"]).to(dev)
    rr = T * min(K, R)
    ws = moe.workspace(T, K, E, R, dev)
    sets = []
    for _ in range(args.sets):
        x = x0.clone()
        o = moe.dedup_dispatch(x, idx, E, R, ws=ws)
        y = o.packed.clone()
        sets.append(dict(x=x, o=o, y=y, out=torch.empty((T, H), dtype=torch.float32, device=dev),
                         ow=torch.empty(T, dtype=torch.float32, device=dev)))
    partial = torch.empty((rr, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    n_recv = int(sets[0]["o"].recv_cnt.sum().item())
    n_rows = int(sets[0]["o"].packed_cnt.sum().item())
    assert int(sets[0]["o"].stats[2].item()) == 0, "recv rows dropped"

    def plan(st, two_stage):
        return dict(R=R, idx=idx, rank_slot=st["o"].rank_slot, recv_rows=rr,
                    partial=partial if two_stage else None)

    def step(st, ev=None, two_stage=False):
        if ev: ev[0].record(stream)
        moe.dedup_dispatch(st["x"], idx, E, R, out=st["o"], ws=ws)
        if ev: ev[1].record(stream)
        moe.combine(st["y"], st["o"].tok_map, w, E=E, out_dtype=torch.float32,
                    dedup=plan(st, two_stage), out=st["out"], out_weights=st["ow"])
        if ev: ev[2].record(stream)

    res = {}
    for two_stage in (False, True):
        for i in range(args.warmup):
            step(sets[i % len(sets)], two_stage=two_stage)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(sets[i % len(sets)], ev[i], two_stage)
        torch.cuda.synchronize()
        tail = lambda v: v[1:] if len(v) > 2 else v
        res[two_stage] = (statistics.median(tail([e[0].elapsed_time(e[2]) * 1e3 for e in ev])),
                          statistics.median(tail([e[0].elapsed_time(e[1]) * 1e3 for e in ev])),
                          statistics.median(tail([e[1].elapsed_time(e[2]) * 1e3 for e in ev])))
    st = sets[0]
    ow_err = float((st["ow"] - 1.0).abs().max().item())
    assert ow_err < 1e-5, ow_err
    del sets, partial
    torch.cuda.empty_cache()
    eb = 4
    row = H * eb
    meta_d = T * K * 4 + T * K * 8 + n_rows * 4 + n_recv * 4 + T * R * 4
    disp_b = T * row + 2 * n_recv * row + n_rows * row + meta_d
    comb_fused = n_rows * row + T * row + T * K * 16 + T * R * 4 + T * 4
    comb_two = comb_fused + 2 * n_recv * row
    gb = lambda b, us: round(b / (us * 1e-6) / 1e9, 1)
    pair_f, disp_f, comb_f = res[False]
    pair_t, disp_t, comb_t = res[True]
    out = {"workload": name, "T": T, "H": H, "E": E, "K": K, "R": R, "dtype": "f32",
           "recv_rows": n_recv, "packed_rows": n_rows,
           "dispatch_us": round(disp_f, 2), "dispatch_gbps": gb(disp_b, disp_f),
           "combine_fused_us": round(comb_f, 2), "combine_fused_gbps": gb(comb_fused, comb_f),
           "pair_fused_us": round(pair_f, 2),
           "pair_fused_pct_hbm_peak": round(100 * (disp_b + comb_fused) / (pair_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
           "combine_two_stage_us": round(comb_t, 2), "combine_two_stage_gbps": gb(comb_two, comb_t),
           "pair_two_stage_us": round(pair_t, 2),
           "pair_two_stage_pct_hbm_peak": round(100 * (disp_b + comb_two) / (pair_t * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
           "algorithmic_bytes": {"dispatch": disp_b, "combine_fused": comb_fused,
                                 "combine_two_stage": comb_two}}
    log(f"[bench] dedup: dispatch {disp_f:.1f} us ({out['dispatch_gbps']} GB/s), combine fused "
        f"{comb_f:.1f} us, two-stage {comb_t:.1f} us; pair {pair_f:.1f} / {pair_t:.1f} us")
    return out


def latency_configs(moe, W, dev, warmup=20, reps=50, names=("tiny", "decode", "prefill")):
    """Latency of the tiny, decode and prefill configurations (parity cases,
    not bench lines): HIP events around each dispatch and combine, one buffer
    set, a sleep kernel queued ahead of each pair so that host launch latency is
    not timed; then the pair captured as one graph and replayed the same way;
    then the host side: time inside each call and the wall clock of a round
    with its synchronisation.  Expert stand-in: identity (the packed rows are
    the combine's input)."""
    import numpy as np
    import torch

    res = {}
    for name in names:
        d = W.make_inputs(name)
        T, H, E, K = d["T"], d["H"], d["E"], d["K"]
        cap = int(np.bincount(d["idx"].ravel(), minlength=E).max()) if d["layout"] == "padded" else 0
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
        idx = torch.from_numpy(d["idx"]).to(dev)
        w = torch.from_numpy(d["w"]).to(dev)
        ws = moe.workspace(T, K, E, 0, dev)
        o = moe.dispatch(x, idx, E, cap=cap, ws=ws)
        y = o.packed.clone()
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ow = torch.empty(T, dtype=torch.float32, device=dev)

        def pair():
            moe.dispatch(x, idx, E, cap=cap, out=o, ws=ws)
            moe.combine(y, o.tok_map, w, out=out, out_weights=ow)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        disp, comb, both = [], [], []
        for i in range(warmup + reps):
            torch.cuda._sleep(2_000_000)
            ev[0].record()
            moe.dispatch(x, idx, E, cap=cap, out=o, ws=ws)
            ev[1].record()
            moe.combine(y, o.tok_map, w, out=out, out_weights=ow)
            ev[2].record()
            torch.cuda.synchronize()
            if i >= warmup:
                disp.append(ev[0].elapsed_time(ev[1]) * 1e3)
                comb.append(ev[1].elapsed_time(ev[2]) * 1e3)
                both.append(ev[0].elapsed_time(ev[2]) * 1e3)
        cs = torch.cuda.Stream(dev)
        cs.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                pair()
        torch.cuda.synchronize()
        graph = []
        for i in range(warmup + reps):
            torch.cuda._sleep(2_000_000)
            ev[0].record()
            g.replay()
            ev[2].record()
            torch.cuda.synchronize()
            if i >= warmup:
                graph.append(ev[0].elapsed_time(ev[2]) * 1e3)
        # host time inside each call (the pages' hdis / hcom) and the host wall
        # clock of a round with its synchronisation (hwal): through the Python
        # binding, and through bare ctypes calls of the C ABI with prepared
        # arguments (what a C caller pays: argument checks and the launches)
        L = moe.load()
        P = moe._lib.ptr
        st_ = moe._lib._stream(dev)
        pk = moe._lib.dtype_code(x.dtype)
        d_args = (P(x), pk, T, H, P(idx), K, E, cap, o.packed.shape[0], P(o.packed), pk, None,
                  P(o.packed_cnt), P(o.packed_off), P(o.packed_src), P(o.tok_map), P(o.stats),
                  P(ws), ws.numel(), st_)
        c_args = (P(y), pk, y.shape[0], H, P(o.tok_map), P(w), T, K, 0, None, P(out), pk, P(ow), st_)
        hd, hc, hw, rd, rc = [], [], [], [], []
        for i in range(warmup + reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            moe.dispatch(x, idx, E, cap=cap, out=o, ws=ws)
            t1 = time.perf_counter()
            moe.combine(y, o.tok_map, w, out=out, out_weights=ow)
            t2 = time.perf_counter()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            u0 = time.perf_counter()
            sd = L.moe_dispatch(*d_args)
            u1 = time.perf_counter()
            sc = L.moe_combine(*c_args)
            u2 = time.perf_counter()
            assert sd == 0 and sc == 0
            if i >= warmup:
                hd.append((t1 - t0) * 1e6)
                hc.append((t2 - t1) * 1e6)
                hw.append((t3 - t0) * 1e6)
                rd.append((u1 - u0) * 1e6)
                rc.append((u2 - u1) * 1e6)
        torch.cuda.synchronize()
        med = lambda v: round(statistics.median(v), 2)
        host = {"dispatch_us": med(hd), "combine_us": med(hc), "round_wall_us": med(hw),
                "dispatch_abi_us": med(rd), "combine_abi_us": med(rc)}
        res[name] = {"T": T, "H": H, "E": E, "K": K, "cap": cap, "dispatch_us": med(disp),
                     "combine_us": med(comb), "pair_us": med(both), "graph_pair_us": med(graph),
                     "pair_us_min": round(min(both), 2), "pair_us_std": round(statistics.pstdev(both), 2),
                     "host_us": host}
        if name == "prefill":   # HBM-bound: also its bandwidth (tiny and decode are latency-bound)
            db, cb = algorithmic_bytes(T, H, K, E, T * K, fp8=False)
            res[name]["algorithmic_bytes"] = {"dispatch": db, "combine": cb}
            for key, us in (("pair", med(both)), ("graph_pair", med(graph))):
                g = (db + cb) / (us * 1e-6) / 1e9
                res[name][f"{key}_gbps"] = round(g, 1)
                res[name][f"{key}_pct_hbm_peak"] = round(100 * g / HBM_PEAK_GBS, 2)
            res[name]["dispatch_gbps"] = round(db / (med(disp) * 1e-6) / 1e9, 1)
            res[name]["combine_gbps"] = round(cb / (med(comb) * 1e-6) / 1e9, 1)
        log(f"[bench] {name}: dispatch {med(disp)} us, combine {med(comb)} us, pair {med(both)} us, "
            f"graph pair {med(graph)} us; host in dispatch {host['dispatch_us']} us "
            f"(bare ABI {host['dispatch_abi_us']}), in combine {host['combine_us']} us "
            f"(bare ABI {host['combine_abi_us']}), round wall {host['round_wall_us']} us")
        del o, y, out, ow, g
        torch.cuda.empty_cache()
    return res


def copy_ceiling(moe, dev, reps=10):
    """GB/s (bytes read + written) of the library's 16-byte streaming copy of
    1 GiB, on the same stream as the kernels."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    stream = torch.cuda.current_stream(dev)
    for _ in range(3):
        moe.copy16(a, b)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        moe.copy16(a, b)
        e[1].record(stream)
    torch.cuda.synchronize()
    us = statistics.median(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
    del a, b
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (us * 1e-6) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=3, help="rotating buffer sets")
    ap.add_argument("--workload", default="skewed_fp8")
    ap.add_argument("--secondary", default="uniform_bf16",
                    help="second workload reported inside the line ('none' to skip)")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay pass")
    ap.add_argument("--no-dedup", action="store_true", help="skip the dedup workload line")
    ap.add_argument("--no-fp8-combine", action="store_true",
                    help="skip the line that feeds the fp8 rows straight to moe_combine_fp8")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-reps", type=int, default=5, help="timed oracle calls per CPU run")
    ap.add_argument("--cpu-child", nargs=3, metavar=("WORKLOAD", "REPS", "THREADS"),
                    help=argparse.SUPPRESS)
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the tiny / decode / prefill latency configurations")
    ap.add_argument("--latency-reps", type=int, default=50)
    ap.add_argument("--latency-names", default="tiny,decode,prefill",
                    help="configurations timed by the latency leg (comma separated)")
    ap.add_argument("--only-dedup", action="store_true", help="only the dedup line (one JSON line)")
    ap.add_argument("--latency-profile-text", nargs=2, metavar=("PROF_DIR", "OUT_DIR"),
                    help="write the text summary of the rocprofv3 run of --latency-configs")
    ap.add_argument("--latency-configs", action="store_true",
                    help="only time the tiny, decode and prefill configurations (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain 1 GiB copy used to scale HBM counters")
    ap.add_argument("--profile-text", nargs=2, metavar=("PROF_DIR", "OUT_DIR"),
                    help="write the text summaries of the rocprofv3 runs listed in PROFILE_RUNS")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE", "OUT"),
                    help="summarize rocprofv3 FETCH_SIZE / WRITE_SIZE csvs into OUT (json)")
    args = ap.parse_args()

    if args.cpu_child:
        cpu_child(args.cpu_child[0], int(args.cpu_child[1]), int(args.cpu_child[2]))
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.profile_text:
        profile_text(*args.profile_text)
        return
    if args.latency_profile_text:
        latency_profile_text(*args.latency_profile_text)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this path is built "
              "and measured on a single GPU; its multi-GPU form is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_moe_route_count_amd as moe
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return
    names = tuple(n for n in args.latency_names.split(",") if n)
    if args.latency_configs:
        print(json.dumps({"latency_configs": latency_configs(moe, W, dev, reps=args.latency_reps,
                                                             names=names)}), flush=True)
        return
    if args.only_dedup:
        print(json.dumps({"dedup": dedup_line(moe, W, args, dev)}), flush=True)
        return
    name = args.workload
    r = measure(moe, W, name, args, dev, graphs=not args.no_graph)
    t_us, d_us, c_us = r["pair_us"], r["dispatch_us"], r["combine_us"]
    disp_b, comb_b = r["disp_b"], r["comb_b"]
    total_b = disp_b + comb_b
    gbs = total_b / (t_us * 1e-6) / 1e9
    comb_gbs = comb_b / (c_us * 1e-6) / 1e9
    disp_gbs = disp_b / (d_us * 1e-6) / 1e9
    c_avg = r["combine_us_mean"]
    roof_gbs = comb_b / (c_avg * 1e-6) / 1e9
    khash = source_hash(COMBINE_SOURCES)
    prof = stored_profile(khash)
    traffic = prof.get("traffic_bytes_per_launch")
    log(f"[bench] dispatch {d_us:.1f} us ({disp_gbs:.0f} GB/s)  combine {c_us:.1f} us "
        f"({comb_gbs:.0f} GB/s)  total {t_us:.1f} us ({gbs:.0f} GB/s, {100 * gbs / HBM_PEAK_GBS:.1f}% "
        f"of peak)  wall {r['wall_ms'] * 1e3:.1f} us/step")

    sec = None
    if args.secondary != "none" and args.secondary != name:
        s2 = measure(moe, W, args.secondary, args, dev, graphs=not args.no_graph)
        tb2 = s2["disp_b"] + s2["comb_b"]
        g2 = tb2 / (s2["pair_us"] * 1e-6) / 1e9
        sec = {"workload": s2["name"], "T": s2["T"], "H": s2["H"], "E": s2["E"], "K": s2["K"],
               "routing": s2["routing"], "payload": "fp8_e4m3+f32_scale_per_128" if s2["fp8"] else "bf16",
               "pair_us": round(s2["pair_us"], 2), "pair_us_min": round(s2["pair_us_min"], 2),
               "pair_us_std": round(s2["pair_us_std"], 2), "dispatch_us": round(s2["dispatch_us"], 2),
               "combine_us": round(s2["combine_us"], 2), "timing_us": s2["timing"],
               "algorithmic_bytes": {"dispatch": s2["disp_b"], "combine": s2["comb_b"]},
               "achieved_gbps": round(g2, 1), "pct_hbm_peak": round(100 * g2 / HBM_PEAK_GBS, 2)}
        if "graph_pair_us" in s2:
            sec["graph_pair_us"] = round(s2["graph_pair_us"], 2)
        log(f"[bench] secondary {s2['name']}: {s2['pair_us']:.1f} us ({g2:.0f} GB/s)")

    f8 = None
    if r["fp8"] and not args.no_fp8_combine:
        s3 = measure(moe, W, name, args, dev, graphs=False, y_fp8=True)
        tb3 = s3["disp_b"] + s3["comb_b"]
        g3 = tb3 / (s3["pair_us"] * 1e-6) / 1e9
        f8 = {"workload": name, "combine": "fp8_e4m3+f32_scale_per_128_in_f32_acc_bf16_out",
              "pair_us": round(s3["pair_us"], 2), "pair_us_min": round(s3["pair_us_min"], 2),
              "pair_us_std": round(s3["pair_us_std"], 2), "dispatch_us": round(s3["dispatch_us"], 2),
              "combine_us": round(s3["combine_us"], 2),
              "algorithmic_bytes": {"dispatch": s3["disp_b"], "combine": s3["comb_b"]},
              "achieved_gbps": round(g3, 1), "pct_hbm_peak": round(100 * g3 / HBM_PEAK_GBS, 2),
              "combine_gbps": round(s3["comb_b"] / (s3["combine_us"] * 1e-6) / 1e9, 1)}
        log(f"[bench] fp8-input combine: pair {s3['pair_us']:.1f} us, combine {s3['combine_us']:.1f} us "
            f"({f8['combine_gbps']:.0f} GB/s)")

    f4 = None
    if r["fp8"] and not args.no_fp8_combine:
        s4 = measure(moe, W, name, args, dev, graphs=False, y_fp8=True, fp4=True)
        tb4 = s4["disp_b"] + s4["comb_b"]
        g4 = tb4 / (s4["pair_us"] * 1e-6) / 1e9
        f4 = {"workload": name, "payload": "fp4_e2m1+f32_scale_per_128",
              "combine": "fp4_e2m1+f32_scale_per_128_in_f32_acc_bf16_out",
              "pair_us": round(s4["pair_us"], 2), "pair_us_min": round(s4["pair_us_min"], 2),
              "dispatch_us": round(s4["dispatch_us"], 2), "combine_us": round(s4["combine_us"], 2),
              "algorithmic_bytes": {"dispatch": s4["disp_b"], "combine": s4["comb_b"]},
              "achieved_gbps": round(g4, 1), "pct_hbm_peak": round(100 * g4 / HBM_PEAK_GBS, 2)}
        log(f"[bench] fp4 payload: pair {s4['pair_us']:.1f} us (dispatch {s4['dispatch_us']:.1f}, "
            f"combine {s4['combine_us']:.1f})")

    dv = None
    if r["fp8"] and not args.no_fp8_combine:
        dv = dispatch_variants(moe, W, name, args, dev)

    dd = None
    if not args.no_dedup:
        dd = dedup_line(moe, W, args, dev)

    copy_gbs = copy_ceiling(moe, dev)
    log(f"[bench] 16-byte streaming copy of 1 GiB: {copy_gbs:.0f} GB/s (read + write)")

    lat = None
    if not args.no_latency:
        lat = latency_configs(moe, W, dev, reps=args.latency_reps, names=names)

    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu oracle baseline on the full {name} workload ...")
        cpu = cpu_baseline(name, r["disp_b"] + r["comb_b"], reps=args.cpu_reps)

    line = {
        "metric": METRIC,
        "value": round(t_us, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "T": r["T"], "H": r["H"], "E": r["E"], "K": r["K"],
                   "routing": "zipf1.2" if r["routing"] == "zipf" else "uniform",
                   "payload": "fp8_e4m3+f32_scale_per_128" if r["fp8"] else "bf16",
                   "combine": "bf16_in_f32_acc_bf16_out", "layout": "compact",
                   "buffer_sets": args.sets,
                   "geometry": moe.geometry(),
                   "dtypes": {"x": "bf16", "payload": "fp8_e4m3" if r["fp8"] else "bf16",
                              "scales": "f32" if r["fp8"] else None, "y": "bf16",
                              "arithmetic": "f32", "accumulate": "f32", "out": "bf16"}},
        "achieved_gbps": round(gbs, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "pct_copy_ceiling": round(100 * gbs / copy_gbs, 2),
        "copy_ceiling_gbps": round(copy_gbs, 1),
        "pair_us_min": round(r["pair_us_min"], 2),
        "pair_us_std": round(r["pair_us_std"], 2),
        "graph_pair_us": round(r["graph_pair_us"], 2) if "graph_pair_us" in r else None,
        "pct_hbm_peak_graph": (round(100 * total_b / (r["graph_pair_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)
                               if "graph_pair_us" in r else None),
        "graph_multi_step_pair_us": (round(r["graph_multi_pair_us"], 2)
                                     if "graph_multi_pair_us" in r else None),
        "pct_hbm_peak_graph_multi_step": (round(100 * total_b / (r["graph_multi_pair_us"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 2)
                                          if "graph_multi_pair_us" in r else None),
        "pct_hbm_peak_wall": round(100 * total_b / (r["wall_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "graph_pair_us_min": round(r["graph_pair_us_min"], 2) if "graph_pair_us" in r else None,
        "dispatch_us": round(d_us, 2),
        "combine_us": round(c_us, 2),
        "dispatch_gbps": round(disp_gbs, 1),
        "timing_us": r["timing"],
        "algorithmic_bytes": {"dispatch": disp_b, "combine": comb_b},
        "roofline": {"bound": "hbm", "kernel": "combine_kernel", "achieved": round(roof_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": comb_b,
                     "avg_launch_us": round(c_avg, 2),
                     "avg_launch_us_source": "HIP events around each combine launch of the timed "
                                             "region, on its stream (includes event overhead)",
                     "kernel_trace": ({"avg_launch_us": round(prof["trace_avg_us"], 2),
                                       "frac": round(comb_b / (prof["trace_avg_us"] * 1e-6) / 1e9
                                                     / HBM_PEAK_GBS, 4),
                                       "source": "profiles/skewed_fp8_headline_kernel_trace.txt "
                                                 "(rocprofv3 kernel trace of this pair alone, same "
                                                 "kernel source)"}
                                      if prof.get("trace_avg_us") else None)},
        "secondary": sec,
        "fp8_combine": f8,
        "fp4_payload": f4,
        "dispatch_variants": dv,
        "dedup": dd,
        "latency_configs": lat,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
