"""LayerNorm-mode activation quantizer against the oracle, every element: row
lengths on both sides of each kernel boundary of the LayerNorm dispatch (one
to four 16-byte chunks per lane of 256 in the two-row kernel, five to eight in
the wide-row kernel, ragged chunk counts), token counts that leave a partial
last sweep of the grid and an odd last row pair, fp32 inputs, and the three
step modes.
Codes, per-token steps and the batch step must match bit for bit.
"""
import numpy as np
import pytest

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

# (M, K, x dtype): K / 8 chunks, ceil(chunks / 256) per lane
CASES = [
    (1, 64, "bf16"),        # 8 chunks
    (2, 512, "bf16"),
    (4097, 512, "bf16"),    # two sweeps of 1024 row pairs, last pair odd
    (3, 2048, "bf16"),      # 256 chunks: one per lane
    (255, 2112, "bf16"),    # 264 chunks: two per lane, ragged
    (2053, 4096, "bf16"),   # past one sweep of 1024 row pairs, last pair odd
    (7, 4160, "bf16"),      # 520 chunks: three per lane
    (130, 6144, "bf16"),
    (2051, 8192, "bf16"),   # four per lane, two sweeps and a ragged tail
    (33, 8256, "bf16"),     # 1032 chunks: the wide-row kernel, six chunks per lane
    (1100, 10240, "bf16"),  # 1280 chunks, five of six per lane; tokens past one sweep of 1024 blocks
    (5, 12288, "bf16"),     # 1536 chunks: six per lane
    (801, 14400, "bf16"),   # 1800 chunks: eight per lane, ragged; tokens past one sweep of 768 blocks
    (9, 16384, "bf16"),     # 2048 chunks: eight per lane
    (65, 4096, "f32"),      # fp32 input: the one-row kernel
    (7, 12288, "f32"),      # fp32 input past 1024 chunks: the one-row kernel
]
MODES = ["per_token", "static", "dynamic_per_tensor"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}")
def test_ln_quantizer_every_element(case, mode):
    M, K, xdt = case
    say(f"[case] ln quantizer M={M} K={K} {xdt} {mode}")
    spec = datagen.random_layer(M, 8, K, seed=9100 + K + M, x_dtype=xdt,
                                n_outliers=max(1, K // 256), T=16, mode=mode, ln=True)
    x = datagen.eval_x(spec)
    gamma, beta = datagen.ln_params(spec)
    a = oracle.colmax(datagen.calibration_x(spec))
    s = oracle.smooth_factor(a, oracle.colmax(datagen.weights(spec)), 0.5)
    gs, bs = oracle.ln_fold(gamma, beta, s)
    st = oracle.static_scale(a, s)

    d = dev()
    static_t = to_dev(np.array([st], np.float32), d) if mode == "static" else None
    xq_t, xs_t = sq.sq_smooth_quantize_act(to_dev(x, d), None, to_dev(gs, d), to_dev(bs, d),
                                           1e-5, mode, static_t)
    q_ref, sc_ref, _ = oracle.smooth_quantize_act(
        x, g_s=gs, b_s=bs, eps=1e-5, static=st if mode == "static" else None,
        dynamic_per_tensor=mode == "dynamic_per_tensor")
    assert_same("xq", to_np(xq_t), q_ref)
    if mode == "per_token":
        assert_same("x_scale", to_np(xs_t), sc_ref)
    elif mode == "dynamic_per_tensor":
        assert_same("x_scale", to_np(xs_t), np.atleast_1d(np.asarray(sc_ref, np.float32)))
