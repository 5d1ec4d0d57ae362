"""Run the library's int8 GEMM on one shape a number of times: a short program
for hardware-counter runs of the GEMM kernels alone.

    rocprofv3 --pmc <counters> --output-format csv -d <dir> -o run -- \
        python3 -m w8a8_int8_gemm_colwise_amd.gemm_run M N K reps

Operands are seeded uniform int8 codes, per-token and per-channel steps in
(0, 1e-3], bf16 output (the benchmark's launch configuration).
"""
import sys

import torch

import w8a8_int8_gemm_colwise_amd as sq


def main():
    M, N, K, reps = (int(v) for v in sys.argv[1:5])
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, generator=g).to(dev)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, generator=g).to(dev)
    xs = torch.rand(M, generator=g).to(dev) * 1e-3
    ws = torch.rand(N, generator=g).to(dev) * 1e-3
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for _ in range(reps):
        sq.sq_gemm_w8a8(xq, xs, wq, ws, out_dtype="bf16", y=y)
    torch.cuda.synchronize()
    print("done", M, N, K, reps, flush=True)


if __name__ == "__main__":
    main()
