"""Build libsq.so (the HIP kernels + C ABI) and libsqprobe.so (the
benchmark's attainable-ceiling probes) for gfx950 with hipcc.

    python -m w8a8_int8_gemm_colwise_amd.build

Every translation unit is compiled with -ffp-contract=off (no silent FMA
contraction in the quantize/dequant arithmetic) and without fast-math; fp32
division and sqrt stay IEEE-correctly rounded (hipcc's default).  Packed fp32
instructions are disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "sq")
LIB = os.path.join(HERE, "libsq.so")
SOURCES = ["abi.hip", "calibrate.hip", "act_quant.hip", "gemm.hip", "robust.hip"]
PROBE_LIB = os.path.join(HERE, "libsqprobe.so")
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # that note is expected, anything else is shown
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
