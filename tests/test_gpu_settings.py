"""GPU parity of the SmoothQuant-O1/O2/O3 settings ([Review] §6.3): per-tensor
weight step with per-token (O1), dynamic per-tensor (O2) or static per-tensor
(O3) activation steps, against the oracle, bit for bit (steps, codes,
accumulators, fp32 and bf16 outputs).

Shapes reach every kernel path: the ping-pong GEMM (K % 128 == 0, M > 64),
the skinny decode GEMM (M <= 64), the register-staged fallback (K % 128 != 0),
the two-sweep weight and activation kernels (K beyond 49152), LayerNorm mode,
and the empty batch / empty weight.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import dev, run_layer, to_np

pytestmark = pytest.mark.gpu

SETTINGS = {"O1": "per_token", "O2": "dynamic_per_tensor", "O3": "static"}

CASES = [
    # M, N, K, x_dtype, w_dtype, ln
    (300, 300, 576, "bf16", "f32", False),       # fallback GEMM (K % 128 != 0)
    (257, 513, 1024, "bf16", "bf16", False),     # ping-pong 256x128, ragged edges
    (65, 1000, 4096, "bf16", "bf16", False),
    (33, 200, 512, "bf16", "bf16", True),        # skinny GEMM, two 32-row tiles, LN
    (1, 33, 256, "f32", "f32", True),
    (5, 96, 24576, "bf16", "bf16", False),
    (40, 700, 16384, "bf16", "f32", False),      # per-tensor weight step: elementwise map
    (4, 40, 133120, "bf16", "bf16", False),      # two-sweep weight and activation kernels
    (70, 130, 8192, "bf16", "bf16", True),
]


@pytest.mark.parametrize("setting", sorted(SETTINGS))
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + ("_ln" if c[5] else ""))
def test_settings_every_element(case, setting):
    M, N, K, xdt, wdt, ln = case
    spec = datagen.random_layer(M, N, K, seed=M * 5 + N + K, x_dtype=xdt, w_dtype=wdt,
                                n_outliers=3, T=max(8, M // 2), alpha=0.5, ln=ln)
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    g = b = None
    if ln:
        g, b = datagen.ln_params(spec)
    r = run_layer(spec, xc, w, x, SETTINGS[setting], w_mode="per_tensor", gamma=g, beta=b)
    assert r["cal"]["w_scale"].numel() == 1


@pytest.mark.parametrize("setting", sorted(SETTINGS))
@pytest.mark.parametrize("l", [0, 3], ids=["qkv", "fc2"])
def test_settings_opt67b_prefill_sampled(l, setting):
    spec = datagen.workload(2).layers[l]
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    r = run_layer(spec, xc, w, x, SETTINGS[setting], w_mode="per_tensor", n_rows=32, n_cols=48,
                  seed=l, out_kinds=("bf16", "i32"))
    # the per-tensor weight step reaches 127 somewhere, not in every row
    wq = r["cal"]["wq"]
    assert int(wq.abs().max()) == 127


@pytest.mark.parametrize("setting", ["O1", "O2"])
def test_settings_decode_m1(setting):
    spec = datagen.workload(3).layers[1]
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec, M=1)
    run_layer(spec, xc, w, x, SETTINGS[setting], w_mode="per_tensor", n_cols=64, seed=3)


@pytest.mark.parametrize("setting", ["O2", "O3"])
def test_settings_ln_pipeline_h8192(setting):
    spec = datagen.workload(5).layers[0]
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    g, b = datagen.ln_params(spec)
    run_layer(spec, xc, w, x, SETTINGS[setting], w_mode="per_tensor", n_rows=16, n_cols=24,
              seed=9, out_kinds=("bf16",), gamma=g, beta=b)


def test_per_tensor_empty_inputs():
    """An empty batch has the dynamic per-tensor step FLOOR/127; an empty
    weight the per-tensor weight step FLOOR/127."""
    d = dev()
    K = 128
    floor_step = np.float32(1e-7) / np.float32(127)
    xq, xs = sq.sq_smooth_quantize_act(torch.empty(0, K, device=d, dtype=torch.bfloat16),
                                       torch.ones(K, device=d), mode="dynamic_per_tensor")
    cal = sq.sq_calibrate(torch.randn(4, K, device=d), torch.empty(0, K, device=d), 0.5,
                          w_mode="per_tensor")
    torch.cuda.synchronize()
    assert to_np(xs)[0] == floor_step
    assert to_np(cal["w_scale"])[0] == floor_step


def test_dynamic_per_tensor_step_is_max_of_token_steps():
    """On the GPU too: the batch step equals the largest per-token step, and
    tokens that attain it get the per-token codes."""
    d = dev()
    spec = datagen.random_layer(200, 64, 2048, seed=77, n_outliers=4, T=64)
    x = datagen.eval_x(spec)
    s = oracle.smooth_factor(oracle.colmax(datagen.calibration_x(spec)),
                             oracle.colmax(datagen.weights(spec)), 0.5)
    xt, st = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(d), torch.from_numpy(s).to(d)
    q_t, dt = sq.sq_smooth_quantize_act(xt, st, mode="dynamic_per_tensor")
    q_p, dp = sq.sq_smooth_quantize_act(xt, st, mode="per_token")
    torch.cuda.synchronize()
    dt, dp = to_np(dt), to_np(dp)
    assert dt[0] == dp.max()
    top = np.flatnonzero(dp == dt[0])
    assert np.array_equal(to_np(q_t)[top], to_np(q_p)[top])
