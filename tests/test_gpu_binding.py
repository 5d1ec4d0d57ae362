"""The Python binding checks every caller-supplied output and scale vector
(shape, dtype, device, contiguity) before anything reaches the library, so a
wrong-sized buffer raises instead of being written out of bounds; correctly
preallocated outputs give the same bits as freshly allocated ones."""
import numpy as np
import pytest
import torch

import datagen
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import dev, to_dev, to_np

pytestmark = pytest.mark.gpu


def _layer(M=96, N=160, K=256, seed=3):
    rng = np.random.default_rng(seed)
    d = dev()
    x = datagen.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    xc = datagen.f32_to_bf16_bits(rng.standard_normal((64, K)).astype(np.float32))
    w = datagen.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    return to_dev(x, d), to_dev(xc, d), to_dev(w, d)


def test_rejects_bad_outputs_and_scales():
    x, xc, w = _layer()
    M, K = x.shape
    N = w.shape[0]
    d = x.device
    cal = sq.sq_calibrate(xc, w, 0.5)
    with pytest.raises(ValueError):
        sq.sq_calibrate(xc, w, 0.5, out={"s": torch.empty(K - 1, device=d)})
    with pytest.raises(ValueError):
        sq.sq_calibrate(xc, w, 0.5, out={"wq": torch.empty((N, K), dtype=torch.int16, device=d)})
    with pytest.raises(ValueError):
        sq.sq_smooth_quantize_act(x, cal["s"], xq=torch.empty((M, K - 64), dtype=torch.int8, device=d))
    with pytest.raises(ValueError):
        sq.sq_smooth_quantize_act(x, cal["s"], x_scale=torch.empty(M - 1, device=d))
    with pytest.raises(ValueError):
        sq.sq_smooth_quantize_act(x, cal["s"][:-64])
    xq, xs = sq.sq_smooth_quantize_act(x, cal["s"])
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"], y=torch.empty((M, N + 1), dtype=torch.bfloat16, device=d))
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"], out_dtype="f32",
                        y=torch.empty((M, N), dtype=torch.bfloat16, device=d))
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8(xq, xs.half(), cal["wq"], cal["w_scale"])
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"][: N // 2])
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8_ex(xq, xs, cal["wq"], cal["w_scale"], bias=torch.zeros(N - 1, device=d))
    with pytest.raises(ValueError):
        sq.sq_gemm_w8a8(xq, xs, cal["wq"].t().contiguous()[:, :K], cal["w_scale"])
    with pytest.raises(ValueError):
        sq.sq_channel_quantile(xc, 0.5, out=torch.empty(K, dtype=torch.float64, device=d))


def test_preallocated_outputs_match():
    x, xc, w = _layer(M=130, N=200, K=384, seed=4)
    M, K = x.shape
    N = w.shape[0]
    d = x.device
    f32 = dict(dtype=torch.float32, device=d)
    fresh = sq.sq_calibrate(xc, w, 0.5)
    pre = {k: torch.full_like(v, 7) for k, v in fresh.items()}
    got = sq.sq_calibrate(xc, w, 0.5, out=pre)
    for k in fresh:
        assert got[k] is pre[k]
        assert torch.equal(got[k], fresh[k]), k
    xq0, xs0 = sq.sq_smooth_quantize_act(x, fresh["s"])
    xq1 = torch.full((M, K), 3, dtype=torch.int8, device=d)
    xs1 = torch.full((M,), 5.0, **f32)
    xq2, xs2 = sq.sq_smooth_quantize_act(x, fresh["s"], xq=xq1, x_scale=xs1)
    assert xq2 is xq1 and xs2 is xs1
    assert torch.equal(xq1, xq0) and torch.equal(xs1, xs0)
    y0 = sq.sq_gemm_w8a8(xq0, xs0, fresh["wq"], fresh["w_scale"], out_dtype="f32")
    y1 = torch.full((M, N), 1.5, **f32)
    assert sq.sq_gemm_w8a8(xq0, xs0, fresh["wq"], fresh["w_scale"], out_dtype="f32", y=y1) is y1
    assert np.array_equal(to_np(y1), to_np(y0))
