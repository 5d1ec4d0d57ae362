"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for s, the maxima, the static scale, the folded LayerNorm
parameters, the int8 weights and activations, their scales, the int32
accumulators, and the fp32 and bf16 outputs (the library's numerical contract
fixes every fp32 operation, so the outputs are reproduced bit for bit, which
is stronger than the 1e-6 relative (fp32) / 2^-8 relative (bf16) tolerance).

Small cases compare every element; the full-size workloads run the GPU path at
full size, in the launch configuration the benchmark times, and compare
sampled tokens and output channels that the oracle computes one by one, plus
size-independent properties on every element.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, c5_inputs, dev, run_layer, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _inputs(spec, M=None, T=None):
    return datagen.calibration_x(spec, T=T), datagen.weights(spec), datagen.eval_x(spec, M=M)


# ---- single linear, CPU-oracle sized: every element ----------------------------

@pytest.mark.parametrize("mode", ["static", "per_token"])
def test_single_linear_512_every_element(mode):
    spec = datagen.workload(1).layers[0]
    xc, w, x = _inputs(spec)
    r = run_layer(spec, xc, w, x, mode)
    if mode == "static":
        # evaluation outliers can exceed the calibration peak: clamp exercised
        say(f"  static-mode saturated codes: {r['sat']}")


# ---- ragged small shapes: several tiles and ragged tails -------------------------

RAGGED = [
    # M, N, K, x_dtype, w_dtype, mode, ln, alpha
    (1, 1, 64, "bf16", "bf16", "per_token", False, 0.5),
    (17, 50, 64, "f32", "f32", "per_token", False, 0.5),
    (100, 129, 192, "bf16", "bf16", "per_token", False, 0.25),
    (300, 300, 576, "bf16", "f32", "static", False, 0.75),
    (257, 513, 1024, "bf16", "bf16", "per_token", False, 0.0),
    (65, 1000, 4096, "bf16", "bf16", "per_token", False, 1.0),
    (129, 384, 2112, "f32", "bf16", "static", False, 0.85),
    (33, 200, 512, "bf16", "bf16", "per_token", True, 0.5),
    (70, 130, 8192, "bf16", "bf16", "static", True, 0.5),
    (40, 64, 640, "f32", "f32", "per_token", True, 0.6),
    (5, 96, 24576, "bf16", "bf16", "per_token", False, 0.5),
    (6, 64, 49152, "bf16", "bf16", "per_token", False, 0.5),
    (7, 96, 36928, "bf16", "bf16", "per_token", False, 0.5),   # 4616 chunks: ragged long rows
    (3, 64, 16384 + 64, "bf16", "bf16", "per_token", True, 0.5),
    (4, 40, 133120, "bf16", "bf16", "per_token", False, 0.5),
    # short-K kernel (whole K in LDS): K = 64, 128, 256 with ragged M and N
    (200, 300, 64, "bf16", "bf16", "per_token", False, 0.5),
    (129, 257, 128, "f32", "bf16", "static", True, 0.5),
    (300, 130, 256, "bf16", "bf16", "per_token", False, 0.5),
    (150, 70, 128, "bf16", "f32", "static", False, 0.5),
    # skinny-M (decode) kernel: one and two 32-row tiles, static scale, ragged N
    (64, 72, 1152, "bf16", "bf16", "static", False, 0.5),
    (1, 33, 256, "f32", "f32", "static", True, 0.5),
    (32, 1056, 2048, "bf16", "bf16", "per_token", False, 0.5),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[3]}_{c[4]}_{c[5]}_{'ln' if c[6] else 'plain'}")
def test_ragged_every_element(case):
    M, N, K, xdt, wdt, mode, ln, alpha = case
    spec = datagen.random_layer(M, N, K, seed=M * 7 + N * 3 + K, x_dtype=xdt, w_dtype=wdt,
                                n_outliers=3, T=max(8, M // 2), alpha=alpha, mode=mode, ln=ln)
    xc, w, x = _inputs(spec)
    g = b = None
    if ln:
        g, b = datagen.ln_params(spec)
    run_layer(spec, xc, w, x, mode, gamma=g, beta=b)


@pytest.mark.parametrize("shape", [(1100, 13000, 256), (777, 3000, 1280), (2049, 4097, 512),
                                   (513, 30000, 384), (257, 33000, 384)],
                         ids=lambda t: "x".join(map(str, t)))
def test_ragged_large_tiles_sampled(shape):
    """Shapes that select the large-tile kernels with ragged edges in M and N
    (the last two: 256x256 tiles over the first columns and 256x128 tiles over
    the rest, in one launch); sampled rows always include the first and last
    token, sampled columns the first and last output channel."""
    M, N, K = shape
    spec = datagen.random_layer(M, N, K, seed=M + N + K, n_outliers=4, T=64)
    xc, w, x = _inputs(spec)
    run_layer(spec, xc, w, x, "per_token", n_rows=40, n_cols=48, seed=M)


# ---- full-size workloads: sampled elements ---------------------------------------

@pytest.mark.parametrize("l", range(4), ids=["qkv", "out_proj", "fc1", "fc2"])
def test_opt67b_prefill_m2048(l):
    spec = datagen.workload(2).layers[l]
    xc, w, x = _inputs(spec)
    r = run_layer(spec, xc, w, x, "per_token", n_rows=48, n_cols=64, seed=l)
    _full_size_properties(r, "per_token")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
@pytest.mark.parametrize("l", range(2), ids=["ffn_up", "ffn_down"])
def test_decode_70b_ffn(M, l):
    spec = datagen.workload(3).layers[l]
    xc, w, x = _inputs(spec, M=M)
    r = run_layer(spec, xc, w, x, "per_token", n_rows=None, n_cols=96, seed=M + l)
    _full_size_properties(r, "per_token")


@pytest.mark.parametrize("l", range(4), ids=["qkv", "out_proj", "fc1", "fc2"])
def test_opt175b_layer_m4096(l):
    spec = datagen.workload(4).layers[l]
    xc, w, x = _inputs(spec)
    r = run_layer(spec, xc, w, x, "per_token", n_rows=24, n_cols=32, seed=10 + l,
                  out_kinds=("bf16", "i32"))
    _full_size_properties(r, "per_token")


@pytest.mark.parametrize("mode", ["static", "per_token"])
@pytest.mark.parametrize("alpha", datagen.ALPHA_SWEEP)
def test_ln_pipeline_h8192_alpha_sweep(alpha, mode):
    spec = datagen.workload(5, alpha=alpha).layers[0]
    d = c5_inputs()
    g, b = d["gb"]
    r = run_layer(spec, d["xc"], d["w"], d["x"], mode, n_rows=16, n_cols=24, seed=int(alpha * 100),
                  out_kinds=("bf16",), gamma=g, beta=b, alpha=alpha)
    _full_size_properties(r, mode)


def _full_size_properties(r, mode):
    """Checks on every element, valid at any size."""
    wq = r["cal"]["wq"]
    # every output channel reaches +-127 at its own peak (the scale is max/127)
    assert int((wq.abs().amax(dim=1) == 127).all()) == 1
    xq = r["xq"]
    assert int(xq.min()) >= -127
    if mode != "static":
        # per-token: every token row reaches +-127
        assert int((xq.abs().amax(dim=1) == 127).all()) == 1
    s = to_np(r["cal"]["s"])
    assert np.all(np.isfinite(s)) and np.all(s > 0)


# ---- determinism and edge cases ---------------------------------------------------

def test_repeat_runs_are_bitwise_identical():
    spec = datagen.workload(2).layers[1]
    xc, w, x = _inputs(spec)
    d = dev()
    xct, wt, xt = to_dev(xc, d), to_dev(w, d), to_dev(x, d)
    outs = []
    for _ in range(3):
        cal = sq.sq_calibrate(xct, wt, 0.5)
        xq, xs = sq.sq_smooth_quantize_act(xt, cal["s"])
        y = sq.sq_gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"], out_dtype="bf16")
        torch.cuda.synchronize()
        outs.append([to_np(t) for t in (cal["s"], cal["wq"], xq, xs, y)])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_empty_sizes_are_noops():
    d = dev()
    K = 128
    w = torch.randn(16, K, device=d).to(torch.bfloat16)
    # T = 0 calibration tokens: a_j = FLOOR
    cal = sq.sq_calibrate(torch.empty(0, K, device=d, dtype=torch.bfloat16), w, 0.5)
    torch.cuda.synchronize()
    assert np.all(to_np(cal["x_absmax"]) == np.float32(1e-7))
    wm = oracle.colmax(to_np(w))
    assert_same("s (T=0)", to_np(cal["s"]), oracle.smooth_factor(np.full(K, 1e-7, np.float32), wm, 0.5))
    # M = 0 activations and GEMM
    xq, xs = sq.sq_smooth_quantize_act(torch.empty(0, K, device=d, dtype=torch.bfloat16), cal["s"])
    y = sq.sq_gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"])
    torch.cuda.synchronize()
    assert y.shape == (0, 16)
    # N = 0 weights
    cal0 = sq.sq_calibrate(torch.randn(4, K, device=d), torch.empty(0, K, device=d), 0.5)
    torch.cuda.synchronize()
    assert np.all(to_np(cal0["w_absmax"]) == np.float32(1e-7))


def test_zero_rows_and_extreme_codes():
    d = dev()
    K = 133120
    # all-zero token row: step = FLOOR/127, every code 0
    x = torch.zeros(2, K, device=d, dtype=torch.bfloat16)
    x[1, 5] = 3.0
    s = torch.ones(K, device=d)
    xq, xs = sq.sq_smooth_quantize_act(x, s)
    torch.cuda.synchronize()
    assert int(xq[0].abs().max()) == 0
    assert to_np(xs)[0] == np.float32(1e-7) / np.float32(127)
    assert int(xq[1, 5]) == 127
    # largest K: accumulators at the int32 edge, exact
    a = torch.full((3, K), 127, dtype=torch.int8, device=d)
    a[1] = -127
    b = torch.full((5, K), -127, dtype=torch.int8, device=d)
    b[2] = 127
    acc = sq.sq_gemm_w8a8(a, None, b, None, out_dtype="i32")
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(to_np(a), to_np(b))
    assert_same("acc at K max", to_np(acc), ref)
    assert int(to_np(acc).min()) == -127 * 127 * K
