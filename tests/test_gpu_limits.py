"""GEMM shapes whose weight codes pass 2^31 bytes (N*K > 2^31): the pipelined and
skinny kernels address their operands with 32-bit offsets, so the launcher
sends such shapes to the register-staged kernel, whose offsets are 64-bit.  The
products of the rows past the 2^31-byte mark (output channels n >= 2^31 / K)
are checked with the rest, bit for bit against the oracle on sampled output
channels (every token), for a prefill-sized and a decode-sized batch.
"""
import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

N, K = 65600, 32768          # N*K = 2_149_580_800 bytes of weight codes
FIRST_PAST = (1 << 31) // K  # first output channel whose codes start at byte 2^31


@pytest.fixture(scope="module")
def weight_codes():
    rng = np.random.default_rng(31)
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    d = dev()
    say(f"  weight codes {N} x {K} ({N * K} bytes) to the GPU")
    wq_d = torch.from_numpy(wq).to(d)
    return wq, ws, wq_d, to_dev(ws, d)


@pytest.mark.parametrize("M", [80, 8], ids=["prefill_m80", "decode_m8"])
def test_weight_codes_past_int32_offsets(weight_codes, M):
    assert N * K > (1 << 31)
    wq, ws, wq_d, ws_d = weight_codes
    d = dev()
    rng = np.random.default_rng(1000 + M)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    xs = rng.uniform(1e-3, 2e-2, M).astype(np.float32)
    say(f"  sq_gemm_w8a8 {M} x {N} x {K}, fp32 out")
    y = sq.sq_gemm_w8a8(to_dev(xq, d), to_dev(xs, d), wq_d, ws_d, "per_token", "f32")
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([
        [0, 1, FIRST_PAST - 1, FIRST_PAST, FIRST_PAST + 1, N - 2, N - 1],
        rng.choice(N, size=57, replace=False)])).astype(np.int64)
    acc = oracle.gemm_i32(xq, wq[cols])
    ref = oracle.dequant(acc, xs, ws[cols])
    got = to_np(y)[:, cols]
    assert_same(f"y[:, sampled] {M}x{N}x{K}", got, ref)
