"""Short text summary of a rocprofv3 --kernel-trace --stats run of the benchmark.

    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 bench.py ... > <log>
    python -m w8a8_int8_gemm_colwise_amd.profsum <dir> <summary.txt> --command "<the rocprofv3 command>" [--log <log>]

Lists every kernel (calls, average / min / max duration, share of GPU time),
then every launch shape, then the mean duration over all GEMM launches next to
the benchmark's own event-timed figure from the same run (its JSON line in
<log>), which must agree.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os

GEMM_KERNELS = ("gemm_pp_kernel", "gemm_pp_mixed_kernel", "gemm_shortk_kernel", "gemm_skinny_kernel", "gemm_kernel")


def short(name: str) -> str:
    n = name.replace("void ", "").replace("sq::(anonymous namespace)::", "")
    n = n.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _one(d: str, pattern: str) -> str:
    f = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not f:
        raise FileNotFoundError(f"{pattern} not found under {d}")
    return f[0]


def summarize(d: str, command: str, log: str | None) -> str:
    stats = list(csv.DictReader(open(_one(d, "*kernel_stats.csv"))))
    trace = list(csv.DictReader(open(_one(d, "*kernel_trace.csv"))))
    out = [f"# rocprofv3 kernel statistics", f"# command: {command}",
           "# grid_x is in threads; durations in microseconds", "",
           f"{'kernel':<64} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in stats:
        out.append(f"{short(r['Name'])[:64]:<64} {r['Calls']:>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                   f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                   f"{float(r['Percentage']):>6.2f}")
    g = collections.defaultdict(list)
    gemm = []
    for r in trace:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        key = (short(r["Kernel_Name"]), r["Grid_Size_X"], r["Workgroup_Size_X"])
        g[key].append(us)
        if any(k in r["Kernel_Name"] for k in GEMM_KERNELS):
            gemm.append(us)
    out += ["", "per launch shape:",
            f"{'kernel':<64} {'grid_x':>8} {'wg':>5} {'calls':>6} {'avg_us':>9}"]
    for k, v in sorted(g.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{k[0][:64]:<64} {k[1]:>8} {k[2]:>5} {len(v):>6} {sum(v) / len(v):>9.2f}")
    if gemm:
        out += ["", f"GEMM launches: {len(gemm)}, mean {sum(gemm) / len(gemm):.2f} us (all launches, "
                    "warmup included)"]
    if log and os.path.exists(log):
        for line in open(log):
            if line.startswith("{"):
                j = json.loads(line)
                r = j.get("roofline", {})
                out.append(f"benchmark (same run, HIP events over the timed steps): {r.get('kernel')} "
                           f"avg_launch_us {r.get('avg_launch_us')}, achieved {r.get('achieved')} "
                           f"{r.get('unit')}; step {j.get('ms_per_step')} ms, value {j.get('value')} "
                           f"{j.get('unit')}")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("dest")
    ap.add_argument("--command", required=True)
    ap.add_argument("--log")
    a = ap.parse_args()
    txt = summarize(a.dir, a.command, a.log)
    with open(a.dest, "w") as f:
        f.write(txt)
    print(txt)


if __name__ == "__main__":
    main()
