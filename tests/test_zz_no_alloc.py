"""sq_channel_quantile_noalloc (include/sq.h): the channel quantile for callers
that cannot allocate, on the library's own per-device scratch.  Checked
through the C ABI against the workspace entry point sq_channel_quantile (and
the oracle's nearest-rank quantile), bit for bit, on two calls in a row -- the
second with a smaller input -- then an empty input and the size limit."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _both(x_host, q, d):
    x = to_dev(x_host, d)
    T, K = x.shape
    out = torch.full((K,), -1.0, dtype=torch.float32, device=d)
    sq.sq_channel_quantile_noalloc(x, q, out)
    ref = sq.sq_channel_quantile(x, q)
    torch.cuda.synchronize()
    return to_np(out), to_np(ref)


def test_noalloc_quantile_matches_the_workspace_call_twice():
    d = dev()
    spec = datagen.workload(5).layers[0]
    x1 = datagen.calibration_x(spec, T=3000)                       # bf16 [3000, 8192]
    say(f"[case] noalloc quantile 1: bf16 {x1.shape} q=0.999")
    got, ref = _both(x1, 0.999, d)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    cols = np.arange(0, x1.shape[1], 37)
    want = oracle.channel_quantile(np.ascontiguousarray(x1[:, cols]), 0.999)
    assert np.array_equal(got[cols].view(np.uint32), want.view(np.uint32))

    rng = np.random.default_rng(9)
    x2 = (rng.standard_normal((500, 1024)) * np.exp(rng.uniform(-3, 3, 1024))).astype(np.float32)
    say(f"[case] noalloc quantile 2 (smaller): fp32 {x2.shape} q=0.5")
    got, ref = _both(x2, 0.5, d)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    want = oracle.channel_quantile(x2, 0.5)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_noalloc_quantile_edges():
    d = dev()
    say("[case] noalloc quantile: T = 0, K at the limit, K above it")
    x0 = torch.empty((0, 128), dtype=torch.bfloat16, device=d)
    out = torch.full((128,), -1.0, dtype=torch.float32, device=d)
    sq.sq_channel_quantile_noalloc(x0, 0.5, out)
    torch.cuda.synchronize()
    assert np.all(to_np(out) == np.float32(1e-7))
    rng = np.random.default_rng(3)
    xk = rng.standard_normal((64, sq.SQ_NOALLOC_MAX_K)).astype(np.float32)
    got, ref = _both(xk, 0.9, d)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    big = torch.zeros((4, sq.SQ_NOALLOC_MAX_K + 64), dtype=torch.float32, device=d)
    outb = torch.empty(sq.SQ_NOALLOC_MAX_K + 64, dtype=torch.float32, device=d)
    with pytest.raises(sq.SQError) as ei:
        sq.sq_channel_quantile_noalloc(big, 0.5, outb)
    assert ei.value.status == 2
