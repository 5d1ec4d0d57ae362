"""Plain-mode activation quantizer with a per-tensor step (static, and the
second pass of the dynamic per-tensor step) against the oracle, every element:
row lengths from one chunk per lane up to the longest supported rows, ragged
chunk counts and token counts, bf16 and fp32 inputs.  Codes and the batch step
must match bit for bit.
"""
import numpy as np
import pytest

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

# (M, K, x dtype)
CASES = [
    (1, 64, "bf16"),
    (37, 576, "bf16"),
    (1000, 4096, "bf16"),
    (129, 4160, "f32"),
    (70, 16384, "bf16"),
    (33, 16448, "bf16"),
    (9, 49152, "bf16"),
    (5, 49152, "f32"),
    (3, 133120, "bf16"),
]
MODES = ["static", "dynamic_per_tensor"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}")
def test_per_tensor_step_quantizer_every_element(case, mode):
    M, K, xdt = case
    say(f"[case] per-tensor step quantizer M={M} K={K} {xdt} {mode}")
    spec = datagen.random_layer(M, 8, K, seed=9300 + K + M, x_dtype=xdt,
                                n_outliers=max(1, K // 512), T=16, mode=mode)
    x = datagen.eval_x(spec)
    a = oracle.colmax(datagen.calibration_x(spec))
    s = oracle.smooth_factor(a, oracle.colmax(datagen.weights(spec)), 0.5)
    # the calibration set has 16 tokens, so the evaluation tokens saturate
    # some codes in static mode: the clamp is exercised
    st = oracle.static_scale(a, s)

    d = dev()
    static_t = to_dev(np.array([st], np.float32), d) if mode == "static" else None
    xq_t, xs_t = sq.sq_smooth_quantize_act(to_dev(x, d), to_dev(s, d), mode=mode,
                                           static_scale=static_t)
    q_ref, sc_ref, _ = oracle.smooth_quantize_act(
        x, s=s, static=st if mode == "static" else None,
        dynamic_per_tensor=mode == "dynamic_per_tensor")
    assert_same("xq", to_np(xq_t), q_ref)
    if mode == "dynamic_per_tensor":
        assert_same("x_scale", to_np(xs_t), np.atleast_1d(np.asarray(sc_ref, np.float32)))
