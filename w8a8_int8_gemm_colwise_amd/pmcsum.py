"""Per-kernel summary of rocprofv3 counter runs (--pmc) of the benchmark.

    rocprofv3 --pmc <counters> --output-format csv -d <dir> -o run -- python3 bench.py ...
    python -m w8a8_int8_gemm_colwise_amd.pmcsum <out.txt> --command "<commands>" <dir> [<dir> ...]

For every (kernel, grid) it lists the mean over dispatches of each counter
(summed over the chip per dispatch) and the mean dispatch duration from the
counter runs' own timestamps, then derived figures where their counters are
present: VALU instructions per lane-element of the activation quantizer
(SQ_INSTS_VALU x 64 / elements of one call, elements from the benchmark's
shapes), VALU issue share SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES, the matrix-core
cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024) and the int8 MFMA operations
(SQ_INSTS_VALU_MFMA_MOPS_I8 counts units of 512; they equal 2 M N K), and for
dispatches over 30 us the clock, MfmaUtil and L2 busy share (GRBM_GUI_ACTIVE,
summed over the 8 XCDs, taken per XCD).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os

from .profsum import short


def load(dirs):
    per = collections.OrderedDict()   # (name, grid) -> {counter: [values]}, "dur": [us]
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            disp = {}
            for r in csv.DictReader(open(f)):
                key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
                did = (f, int(r["Dispatch_Id"]))
                e = disp.setdefault(did, {"key": key, "c": collections.defaultdict(float),
                                          "dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
                e["c"][r["Counter_Name"]] += float(r["Counter_Value"])
            for e in disp.values():
                k = per.setdefault(e["key"], {"dur": [], "c": collections.defaultdict(list)})
                k["dur"].append(e["dur"])
                for n, v in e["c"].items():
                    k["c"][n].append(v)
    return per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("out")
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--command", required=True)
    ap.add_argument("--kernels", default="act_quant,gemm_pp,gemm_shortk,gemm_skinny,colmax,weight_quant,smooth_factor")
    ap.add_argument("--elements", default="",
                    help="kernel:grid:elements triples for VALU per element (kernel = a "
                         "substring of its name), e.g. act_quant:524288:8388608")
    a = ap.parse_args()
    per = load(a.dirs)
    elems = [(k, int(g), int(e)) for k, g, e in (p.split(":") for p in a.elements.split(",") if p)]
    want = a.kernels.split(",")
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    lines = ["# rocprofv3 counter summary (per dispatch means)", f"# command: {a.command}", ""]
    for (name, grid), k in per.items():
        if not any(w in name for w in want):
            continue
        c = {n: mean(v) for n, v in k["c"].items()}
        lines.append(f"{name}  grid={grid}  dispatches={max(len(v) for v in k['c'].values())}  "
                     f"mean_us={mean(k['dur']):.2f}")
        for n in sorted(c):
            lines.append(f"    {n:32s} {c[n]:16.1f}")
        n_el = next((e for kk, g, e in elems if kk in name and g == grid), None)
        if "SQ_INSTS_VALU" in c and n_el:
            lines.append(f"    -> VALU instructions per element   {c['SQ_INSTS_VALU'] * 64 / n_el:.2f}")
        if "SQ_ACTIVE_INST_VALU" in c and c.get("SQ_WAVE_CYCLES"):
            lines.append(f"    -> VALU issue / wave cycles        {c['SQ_ACTIVE_INST_VALU'] / c['SQ_WAVE_CYCLES']:.3f}")
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            # the matrix-core cycles summed over the 1024 SIMDs; at 2048 int8
            # ops per SIMD cycle they equal ops / 2048: the cycles the work
            # needs, against the dispatch duration at a given clock
            per_simd = c["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
            lines.append(f"    -> MFMA cycles per SIMD            {per_simd:.0f} "
                         f"(= {per_simd / (mean(k['dur']) * 1e3):.3f} of the dispatch at 1 GHz)")
        if c.get("GRBM_GUI_ACTIVE") and mean(k["dur"]) > 30:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs: per XCD it counts the
            # busy cycles at the shader clock (dispatches long enough that the
            # dispatch time stamps and the busy window agree)
            cyc = c["GRBM_GUI_ACTIVE"] / 8
            lines.append(f"    -> clock (GRBM per XCD / duration) {cyc / (mean(k['dur']) * 1e3):.2f} GHz")
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                lines.append(f"    -> MfmaUtil (MFMA cycles / (cycles x 1024 SIMDs)) "
                             f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.3f}")
            if c.get("TCC_BUSY_sum"):
                lines.append(f"    -> L2 busy (TCC_BUSY / (cycles x 128 channels)) "
                             f"{c['TCC_BUSY_sum'] / (cyc * 128):.3f}")
        if c.get("SQ_INSTS_VALU_MFMA_MOPS_I8"):
            lines.append(f"    -> int8 MFMA ops                   {c['SQ_INSTS_VALU_MFMA_MOPS_I8'] * 512:.4e}")
        lines.append("")
    open(a.out, "w").write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
