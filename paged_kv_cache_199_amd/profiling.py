"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m paged_kv_cache_199_amd.profiling stats <run_kernel_stats.csv> <out.txt> "<command>"
    python -m paged_kv_cache_199_amd.profiling traffic <bench_log> <fetch_dir> <write_dir> \\
        <copy_fetch_dir> <copy_write_dir> "<commands>"

`traffic` reads FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the partition kernel that the bench
line in <bench_log> names from two counter runs, scales each by what the same counter reads for a
plain device copy of known size (the calibration run of `bench.py --calibrate-copy`: 1 GiB read,
1 GiB written per launch), and writes profiles/traffic_<path>_<schedule>_<workload>.json with the
launch configuration and the kernel-source hash, both of which bench.py checks before it reports the
figure.
"""
from __future__ import annotations

import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30                     # bench.py --calibrate-copy: 2^28 fp32 per launch
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_stats(csv_path):
    rows = list(csv.DictReader(open(csv_path)))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                    "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                    "pct": float(r["Percentage"])})
    return out


def short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")[:90]


def write_stats(csv_path, out_txt, command):
    st = kernel_stats(csv_path)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {command}", "",
             f"{'kernel':92s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'%time':>7s}"]
    for r in st:
        lines.append(f"{short(r['name']):92s} {r['calls']:6d} {r['avg_ns'] / 1e3:10.2f} "
                     f"{r['min_ns'] / 1e3:10.2f} {r['max_ns'] / 1e3:10.2f} {r['pct']:7.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    return out_txt


def counter_means(run_dir, counter):
    vals = defaultdict(list)
    for root, _, files in os.walk(run_dir):
        for f in files:
            if f.endswith("counter_collection.csv"):
                for r in csv.DictReader(open(os.path.join(root, f))):
                    if r["Counter_Name"] == counter:
                        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def pick(means, substr):
    hits = [v for k, v in means.items() if substr in k]
    if not hits:
        raise KeyError(f"no kernel matching {substr!r}")
    return hits[0]


def bench_line(log):
    for line in reversed(open(log).read().strip().splitlines()):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise ValueError(f"no bench line in {log}")


def write_traffic(bench_log, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    sys.path.insert(0, ROOT)
    import bench

    b = bench_line(bench_log)
    cfg = b["config"]
    kernel_sub = "pkv::" + b["roofline"]["kernel"] + "<"
    workload, path, schedule = cfg["workload"], cfg["path"], cfg["schedule"]

    fetch = pick(counter_means(fetch_dir, "FETCH_SIZE"), kernel_sub)
    write = pick(counter_means(write_dir, "WRITE_SIZE"), kernel_sub)
    cf = pick(counter_means(copy_fetch_dir, "FETCH_SIZE"), COPY_KERNEL)
    cw = pick(counter_means(copy_write_dir, "WRITE_SIZE"), COPY_KERNEL)
    f_scale = COPY_BYTES / (cf * 1024)
    w_scale = COPY_BYTES / (cw * 1024)
    d = {
        "workload": workload, "path": path, "schedule": schedule, "kernel": b["roofline"]["kernel"],
        "partition_size": cfg["partition_size"], "pipeline_depth": cfg["pipeline_depth"],
        "grid_waves": cfg["grid_waves"],
        "algorithmic_bytes_per_launch": b["roofline"]["algorithmic_bytes_per_launch"],
        "fetch_kib_per_dispatch": round(fetch, 1), "write_kib_per_dispatch": round(write, 1),
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "bytes_per_launch": int(round(fetch * 1024 * f_scale + write * 1024 * w_scale)),
        "read_bytes_per_launch": int(round(fetch * 1024 * f_scale)),
        "write_bytes_per_launch": int(round(write * 1024 * w_scale)),
        "source_hash": bench.kernel_source_hash(),
        "commands": commands,
    }
    d["traffic_over_algorithmic"] = round(d["bytes_per_launch"] / d["algorithmic_bytes_per_launch"], 4)
    out = os.path.join(PROFILES, f"traffic_{path}_{schedule}_{workload}.json")
    json.dump(d, open(out, "w"), indent=1)
    return out


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        print(write_stats(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif mode == "traffic":
        print(write_traffic(*sys.argv[2:8]))
    else:
        raise SystemExit(f"unknown mode {mode}")
