"""GPU parity of the fused GEMM epilogue (sq_gemm_w8a8_ex): bias, ReLU, and
int8 output requantized for the next linear ([Edge] §二: no separate runtime
operator between two int8 GEMMs), against the oracle, bit for bit; plus the
equivalence of the fused int8 output with the unfused graph (fp32 output,
then the static-mode activation quantizer) and an OPT-6.7B-shaped
fc1 -> ReLU -> fc2 chain at full size with the fc2 quantizer fused away.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, sample_idx, say, to_dev, to_np

pytestmark = pytest.mark.gpu

SHAPES = [
    # M, N, K: ping-pong 256x128 and 256x256 tiles, short K (K = 128, 256), skinny (M <= 64),
    # fallback (K % 128 != 0);
    # N a multiple of 64 where the unfused graph is compared too
    (257, 513, 1024),
    (300, 1100, 256),
    (200, 320, 128),
    (290, 2048, 512),
    (64, 200, 512),
    (1, 96, 2048),
    (40, 192, 1152),
    (130, 150, 576),
    (130, 320, 576),
]


def _layer(M, N, K, seed):
    spec = datagen.random_layer(M, N, K, seed=seed, n_outliers=3, T=max(8, M // 2))
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    cal = oracle.calibrate(xc, w, spec.alpha)
    xq, xs, _ = oracle.smooth_quantize_act(x, s=cal["s"])
    return spec, cal, xq, xs


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t)))
def test_fused_bias_relu_every_element(shape, relu):
    M, N, K = shape
    spec, cal, xq, xs = _layer(M, N, K, seed=M + 3 * N + K)
    b = datagen.bias(spec)
    d = dev()
    args = (to_dev(xq, d), to_dev(xs, d), to_dev(cal["wq"], d), to_dev(cal["w_scale"], d))
    say(f"[case] fused bias relu={relu} M={M} N={N} K={K}")
    for out in ("f32", "bf16"):
        y = sq.sq_gemm_w8a8_ex(*args, out_dtype=out, bias=to_dev(b, d), relu=relu)
        torch.cuda.synchronize()
        ref = oracle.gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"], out=out, bias=b, relu=relu)
        assert_same(f"y[{out}]", to_np(y), ref)
    if relu:
        assert float(y.float().min()) >= 0.0


@pytest.mark.parametrize("with_s", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda t: "x".join(map(str, t)))
def test_fused_requant_every_element_and_equals_unfused(shape, with_s):
    """int8 codes for the next linear = oracle; and = the unfused graph on the
    GPU (fp32 output with the same epilogue, then sq_smooth_quantize_act in
    static mode with s = next_s)."""
    M, N, K = shape
    spec, cal, xq, xs = _layer(M, N, K, seed=7 * M + N + K)
    b = datagen.bias(spec)
    rng = np.random.default_rng(M + N)
    ns = rng.uniform(0.1, 8.0, N).astype(np.float32) if with_s else None
    # a step that saturates a few of the largest outputs
    y32 = oracle.epilogue(oracle.dequant(oracle.gemm_i32(xq, cal["wq"]), xs, cal["w_scale"]),
                          b, relu=True)
    xh = y32 if ns is None else oracle.act_smooth(y32, ns)
    step = np.float32(np.abs(xh).max() / 150.0)
    d = dev()
    args = (to_dev(xq, d), to_dev(xs, d), to_dev(cal["wq"], d), to_dev(cal["w_scale"], d))
    st_t = torch.tensor([step], device=d)
    ns_t = None if ns is None else to_dev(ns, d)
    say(f"[case] fused requant s'={with_s} M={M} N={N} K={K}")
    q = sq.sq_gemm_w8a8_ex(*args, out_dtype="i8", bias=to_dev(b, d), relu=True, next_s=ns_t,
                           next_scale=st_t)
    torch.cuda.synchronize()
    ref, sat = oracle.requant(y32, ns, step)
    assert sat > 0
    assert_same("codes", to_np(q), ref)
    if N % 64 == 0:  # the activation quantizer needs its K (= N here) to be a multiple of 64
        yf = sq.sq_gemm_w8a8_ex(*args, out_dtype="f32", bias=to_dev(b, d), relu=True)
        q_unfused, _ = sq.sq_smooth_quantize_act(yf, ns_t if ns_t is not None else
                                                 torch.ones(N, device=d), mode="static",
                                                 static_scale=st_t)
        torch.cuda.synchronize()
        assert_same("codes vs unfused", to_np(q), to_np(q_unfused))


def test_fused_ffn_chain_opt67b():
    """fc1 (4096 -> 16384) with ReLU whose int8 output is fc2's input codes for
    fc2's smoothing factor and static step, then fc2 (16384 -> 4096): the fc2
    activation quantizer is fused into fc1's epilogue.  Sampled tokens are
    checked through both GEMMs against the oracle chain."""
    wl = datagen.workload(2)
    fc1, fc2 = wl.layers[2], wl.layers[3]
    d = dev()
    c1 = oracle.calibrate(datagen.calibration_x(fc1), datagen.weights(fc1), fc1.alpha)
    c2 = oracle.calibrate(datagen.calibration_x(fc2), datagen.weights(fc2), fc2.alpha)
    x = datagen.eval_x(fc1)
    M = x.shape[0]
    rows = sample_idx(M, 24, 5)
    b1 = datagen.bias(fc1)
    xq1, xs1, _ = oracle.smooth_quantize_act(x, s=c1["s"])
    say("[case] fused fc1->fc2 chain, M=2048")
    q_fc2 = sq.sq_gemm_w8a8_ex(to_dev(xq1, d), to_dev(xs1, d), to_dev(c1["wq"], d),
                               to_dev(c1["w_scale"], d), out_dtype="i8", bias=to_dev(b1, d),
                               relu=True, next_s=to_dev(c2["s"], d),
                               next_scale=torch.tensor([c2["static_scale"]], device=d))
    y2 = sq.sq_gemm_w8a8(q_fc2, torch.tensor([c2["static_scale"]], device=d), to_dev(c2["wq"], d),
                         to_dev(c2["w_scale"], d), mode="static", out_dtype="bf16")
    torch.cuda.synchronize()
    # oracle on the sampled tokens
    acc1 = oracle.gemm_i32(xq1[rows], c1["wq"])
    h = oracle.epilogue(oracle.dequant(acc1, xs1[rows], c1["w_scale"]), b1, relu=True)
    q_ref, sat = oracle.requant(h, c2["s"], c2["static_scale"])
    say(f"  fc2 codes saturated: {sat}")
    assert_same("fc2 codes", to_np(q_fc2)[rows], q_ref)
    y_ref = oracle.gemm_w8a8(q_ref, np.array([c2["static_scale"]], np.float32), c2["wq"],
                             c2["w_scale"], per_token=False, out="bf16")
    assert_same("fc2 output", to_np(y2)[rows], y_ref)
