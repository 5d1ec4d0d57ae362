"""Binding of libsqprobe.so: attainable-ceiling probes for the benchmark.

The roofline fractions in the benchmark are quoted against MI355X's published
peaks (int8 MFMA 5.0 POP/s, HBM3E 8 TB/s).  These probes measure what the
machine attains for the same operations -- a loop of int8 MFMAs on
bell-shaped int8 operands (the shape of quantized activations and weights)
and a streaming read / copy of buffers larger than the last-level cache --
so that a kernel's distance from the attainable value can be told apart from
the machine's own distance to the spec.  See include/sq_probe.h.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsqprobe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; run python -m w8a8_int8_gemm_colwise_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.sqp_mfma_i8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
        L.sqp_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p]
        L.sqp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p]
        for f in (L.sqp_mfma_i8, L.sqp_read, L.sqp_copy):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed to launch (code {rc})")


def _best_ms(torch, stream, fn, reps: int) -> float:
    fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def mfma_i8_tops(dev, blocks: int = 1024, iters: int = 4096, reps: int = 5, seed: int = 7) -> float:
    """Sustained int8 MFMA throughput (TOPS) on operands rne(N(0, 40^2)) clipped
    to [-127, 127]."""
    import torch
    rng = np.random.default_rng(seed)
    ops_src = np.clip(np.rint(rng.normal(0.0, 40.0, size=blocks * 256 * 256)), -127, 127)
    src = torch.from_numpy(ops_src.astype(np.int8)).to(dev)
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    L = lib()

    def run():
        _check(L.sqp_mfma_i8(src.data_ptr(), blocks, iters, out.data_ptr(), stream.cuda_stream),
               "sqp_mfma_i8")

    ms = _best_ms(torch, stream, run, reps)
    ops = blocks * 4 * iters * 4 * 2.0 * 32 ** 3
    return ops / (ms * 1e-3) / 1e12


def hbm_read_gbs(dev, nbytes: int = 1 << 30, blocks: int = 2048, reps: int = 5) -> float:
    """Streaming read bandwidth (GB/s) of a buffer 4x the last-level cache."""
    import torch
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    L = lib()

    def run():
        _check(L.sqp_read(buf.data_ptr(), nbytes, blocks, out.data_ptr(), stream.cuda_stream),
               "sqp_read")

    ms = _best_ms(torch, stream, run, reps)
    return nbytes / (ms * 1e-3) / 1e9


def copy(dev, src, dst, nbytes: int, blocks: int = 2048):
    """Enqueue one plain copy of nbytes from src to dst (torch tensors)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    _check(lib().sqp_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, stream.cuda_stream),
           "sqp_copy")


def hbm_copy_gbs(dev, nbytes: int = 512 << 20, blocks: int = 2048, reps: int = 5) -> float:
    """Copy bandwidth (GB/s, read + written bytes) of 512 MiB buffers."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = _best_ms(torch, stream, lambda: copy(dev, src, dst, nbytes, blocks), reps)
    return 2 * nbytes / (ms * 1e-3) / 1e9
