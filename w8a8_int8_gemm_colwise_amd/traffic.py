"""HBM bytes per GEMM launch from two rocprofv3 counter runs of the benchmark.

The hardware counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count the
bytes the L2 exchanges with HBM.  Their scale is checked on a plain copy of
known size that the benchmark runs when given --traffic-probe (libsqprobe's
copy_kernel, 256 MiB read + 256 MiB written): factor = counter bytes / known
bytes, and every GEMM dispatch's counters are divided by that factor.  Each
counter needs a run of its own (a --pmc pass holds one of them):

    rocprofv3 --pmc FETCH_SIZE -d <dir_fetch> -o run --output-format csv -- \
        python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-probes --traffic-probe
    rocprofv3 --pmc WRITE_SIZE -d <dir_write> -o run --output-format csv -- \
        python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-probes --traffic-probe
    python -m w8a8_int8_gemm_colwise_amd.traffic <dir_fetch> <dir_write>

writes profiles/traffic.json (read by bench.py while gemm.hip is unchanged)
and a text summary beside it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import OrderedDict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GEMM_SRC = os.path.join(HERE, "csrc", "gemm.hip")
COPY_BYTES = 256 << 20
GEMM_KERNELS = ("gemm_pp_kernel", "gemm_pp_mixed_kernel", "gemm_shortk_kernel", "gemm_skinny_kernel", "gemm_kernel")


def _dispatches(d: str, counter: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    out = OrderedDict()
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = int(r["Dispatch_Id"])
            e = out.setdefault(k, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "kib": 0.0})
            e["kib"] += float(r["Counter_Value"])
    return OrderedDict(sorted(out.items()))


def _short(name: str) -> str:
    for g in GEMM_KERNELS:
        i = name.find(g)
        if i >= 0:
            j = name.find("(", i)
            return name[i:j if j > 0 else None]
    return name[:60]


def analyse(dir_fetch: str, dir_write: str):
    fetch = _dispatches(dir_fetch, "FETCH_SIZE")
    write = _dispatches(dir_write, "WRITE_SIZE")
    cf = [v["kib"] * 1024 for v in fetch.values() if "copy_kernel" in v["name"]]
    cw = [v["kib"] * 1024 for v in write.values() if "copy_kernel" in v["name"]]
    if not cf or not cw:
        raise RuntimeError("the runs hold no copy_kernel dispatch (run the benchmark with --traffic-probe)")
    ff = cf[0] / COPY_BYTES
    fw = cw[0] / COPY_BYTES
    gf = [v for v in fetch.values() if any(g in v["name"] for g in GEMM_KERNELS)]
    gw = [v for v in write.values() if any(g in v["name"] for g in GEMM_KERNELS)]
    if not gf or len(gf) != len(gw):
        raise RuntimeError(f"GEMM dispatch counts differ between the runs ({len(gf)} vs {len(gw)})")
    launches = []
    for a, b in zip(gf, gw):
        launches.append({"kernel": _short(a["name"]), "grid": a["grid"],
                         "fetch_bytes": a["kib"] * 1024 / ff, "write_bytes": b["kib"] * 1024 / fw})
    per_launch = sum(x["fetch_bytes"] + x["write_bytes"] for x in launches) / len(launches)
    return {
        "gemm_source_sha256": hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest(),
        "gemm_bytes_per_launch": per_launch,
        "fetch_factor": ff,
        "write_factor": fw,
        "copy_bytes_each_way": COPY_BYTES,
        "gemm_launches": launches,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir_fetch")
    ap.add_argument("dir_write")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--summary", default=os.path.join(ROOT, "profiles",
                                                      "gemm_traffic_opt6.7b_prefill_m2048.txt"))
    ap.add_argument("--command", default="", help="the profiled command, recorded in the summary")
    args = ap.parse_args()
    t = analyse(args.dir_fetch, args.dir_write)
    with open(args.out, "w") as f:
        json.dump(t, f, indent=1)
    lines = [
        "HBM traffic of the GEMM launches (rocprofv3 FETCH_SIZE / WRITE_SIZE, one pass each)",
        f"profiled command: {args.command}" if args.command else "",
        f"counter scale from copy_kernel ({COPY_BYTES >> 20} MiB each way): "
        f"FETCH_SIZE x{t['fetch_factor']:.4f}, WRITE_SIZE x{t['write_factor']:.4f}",
        f"{'kernel':60s} {'grid':>9s} {'fetch MB':>10s} {'write MB':>10s}",
    ]
    for x in t["gemm_launches"]:
        lines.append(f"{x['kernel'][:60]:60s} {x['grid']:9d} {x['fetch_bytes'] / 1e6:10.2f} "
                     f"{x['write_bytes'] / 1e6:10.2f}")
    lines.append(f"mean HBM bytes per GEMM launch: {t['gemm_bytes_per_launch'] / 1e6:.2f} MB")
    with open(args.summary, "w") as f:
        f.write("\n".join(ln for ln in lines if ln) + "\n")
    print("\n".join(ln for ln in lines if ln))


if __name__ == "__main__":
    main()
