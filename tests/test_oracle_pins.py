"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types an oracle formula: each compares against a value
the pages print (tests/golden, cited there), a closed form, an invariant, a
library routine, or brute force on tiny inputs.  Every check is chosen so that
a plausible slip (a swapped exponent, a multiply for a divide, a transposed
operand, a wrong scale axis, round-half-away, a -128 clamp) fails it.
"""
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals, cases = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = [t.strip() for t in line.split("=", 1)]
            if k == "case":
                cases.append(v)
            else:
                vals[k] = float(v)
    return vals, cases


def f32(x):
    return np.asarray(x, dtype=np.float32)


def ulp(x):
    x = np.abs(f32(x))
    return np.spacing(x)


# ---- eq. (3) direction and the worked examples --------------------------------

def test_worked_example_s10():
    """[Teach] §三: peaks 120 / 0.12 with s = 10 become 12 / 1.2, product kept."""
    g, _ = _golden("worked_example_s10.txt")
    x = f32([[g["act_peak"]], [-0.5 * g["act_peak"]]])        # 2 tokens, 1 channel
    w = f32([[g["weight_peak"]], [-0.25 * g["weight_peak"]]])  # 2 outputs, 1 channel
    s = f32([g["s"]])
    xhat = oracle.act_smooth(x, s)
    assert np.abs(xhat).max() == np.float32(g["smoothed_act_peak"])
    # the smoothed weight peak is recovered from the row-0 scale: 127 * d_0 = peak
    wq, wsc = oracle.weight_quant(w, s)
    assert wq[0, 0] == 127
    assert abs(float(wsc[0]) * 127.0 - g["smoothed_weight_peak"]) <= 2 * float(ulp(1.2))
    # the LayerNorm fold divides gamma and beta (activation side of the rewrite)
    gs, bs = oracle.ln_fold(f32([g["act_peak"]]), f32([g["act_peak"]]), s)
    assert gs[0] == np.float32(g["smoothed_act_peak"]) and bs[0] == gs[0]
    # products unchanged in fp64 (eq. (3))
    y = oracle.ref_linear_f64(x, w)
    yh = oracle.ref_smoothed_linear_f64(x, w, s)
    np.testing.assert_allclose(yh, y, rtol=1e-12, atol=0)
    assert abs(y[0, 0] - g["product"]) < 1e-5


def test_toy_example_s50():
    """[Review] §5.4: channel 1 at 100, others 1..3; /50 on X and *50 on W."""
    g, _ = _golden("toy_example_s50.txt")
    rng = np.random.default_rng(7)
    K = 8
    x = rng.uniform(g["other_lo"], g["other_hi"], size=(16, K)).astype(np.float32)
    x[3, 1] = g["outlier_peak"]
    s = np.ones(K, np.float32)
    s[1] = g["s_outlier"]
    xhat = oracle.act_smooth(x, s)
    assert np.abs(xhat[:, 1]).max() == np.float32(g["smoothed_outlier_peak"])
    # other channels untouched (s = 1 is an exact identity)
    np.testing.assert_array_equal(xhat[:, [0, 2, 3, 4, 5, 6, 7]], x[:, [0, 2, 3, 4, 5, 6, 7]])
    w = rng.normal(0, 0.02, size=(5, K)).astype(np.float32)
    np.testing.assert_allclose(oracle.ref_smoothed_linear_f64(x, w, s),
                               oracle.ref_linear_f64(x, w), rtol=1e-12, atol=1e-15)


# ---- eq. (4) -------------------------------------------------------------------

def test_alpha_half_closed_form():
    """Eq. (4) at alpha = 0.5 reduces to sqrt(a / w) (golden, derived by hand)."""
    g, _ = _golden("alpha_half_example.txt")
    s = oracle.smooth_factor(f32([120.0]), f32([0.12]), g["alpha"])
    assert abs(float(s[0]) / g["s"] - 1) < 1e-7
    xhat_peak = np.float32(120.0) / s[0]
    w_peak = np.float32(0.12) * s[0]
    assert abs(float(xhat_peak) / g["smoothed_peak"] - 1) < 1e-6
    assert abs(float(w_peak) / g["smoothed_peak"] - 1) < 1e-6


@pytest.mark.parametrize("alpha", datagen.ALPHA_SWEEP + (0.1, 0.6, 0.9))
def test_eq4_product_forms(alpha):
    """a/s = (a w)^(1-alpha) and w s = (a w)^alpha: a swapped exponent, an
    inverted ratio or a missing power fails this for alpha != 0.5."""
    rng = np.random.default_rng(11)
    a = rng.uniform(0.05, 120.0, 4096).astype(np.float32)
    w = rng.uniform(1e-3, 0.2, 4096).astype(np.float32)
    s = oracle.smooth_factor(a, w, alpha).astype(np.float64)
    al = float(np.float32(alpha))  # the call takes alpha as fp32
    aw = a.astype(np.float64) * w.astype(np.float64)
    # fp32 rounding of s: relative error <= 2^-24
    np.testing.assert_allclose(a / s, aw ** (1 - al), rtol=2 ** -23)
    np.testing.assert_allclose(w * s, aw ** al, rtol=2 ** -23)


def test_alpha_one_flattens_activation_channels():
    """[Edge] §一.2 and [Review] §5.3: alpha = 1 puts every smoothed activation
    channel peak at exactly 1 (exact under the division reading)."""
    spec = datagen.workload(1).layers[0]
    xc = datagen.calibration_x(spec)
    w = datagen.weights(spec)
    a, wm = oracle.colmax(xc), oracle.colmax(w)
    s = oracle.smooth_factor(a, wm, 1.0)
    np.testing.assert_array_equal(s, a)
    peaks = oracle.colmax(oracle.act_smooth(xc, s))
    np.testing.assert_array_equal(peaks, np.ones_like(peaks))
    assert oracle.static_scale(a, s) == np.float32(1.0) / np.float32(127.0)


def test_alpha_zero_normalises_weight_channels():
    """Eq. (4) at alpha = 0: s = 1/w, so every smoothed weight channel peak is 1."""
    rng = np.random.default_rng(3)
    a = rng.uniform(0.1, 100, 2048).astype(np.float32)
    w = rng.uniform(1e-4, 0.5, 2048).astype(np.float32)
    s = oracle.smooth_factor(a, w, 0.0)
    prod = w * s
    assert np.all(np.abs(prod - 1) <= np.spacing(np.float32(1.0)))


@pytest.mark.parametrize("alpha", datagen.ALPHA_SWEEP)
def test_smooth_factor_quad_audit(alpha):
    """fp64 pow/pow/divide rounds to the same fp32 as a quad-precision route;
    no channel of a workload-shaped vector sits near an fp32 rounding tie."""
    spec = datagen.workload(2).layers[0]
    a = oracle.colmax(datagen.calibration_x(spec))
    rng = np.random.default_rng(5)
    w = rng.uniform(0.05, 0.1, spec.K).astype(np.float32)
    near, mism = oracle.smooth_factor_audit(a, w, alpha)
    assert mism == 0 and near == 0


def test_colmax_matches_library_max():
    x = datagen.calibration_x(datagen.workload(2).layers[1])
    ref = np.maximum(np.abs(datagen.bf16_bits_to_f32(x)).max(axis=0), oracle.FLOOR)
    np.testing.assert_array_equal(oracle.colmax(x), ref)
    z = np.zeros((3, 64), np.float32)
    np.testing.assert_array_equal(oracle.colmax(z), np.full(64, oracle.FLOOR, np.float32))


# ---- quantizer ([Review] §2.2) ---------------------------------------------------

def test_quantizer_ties_round_to_even_and_bound():
    d = 1.0  # row peak 127 gives a step of exactly 1
    row = f32([127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5, 2.4999998, -126.5])
    q, sc = oracle.quant_per_token(row[None, :])
    assert sc[0] == np.float32(d)
    np.testing.assert_array_equal(q[0], [127, 2, 4, -2, 0, 2, 0, -2, 2, -126])


def test_quantizer_error_bound_and_symmetric_clamp():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1, size=(64, 1024)).astype(np.float32)
    x[:, 17] *= 60
    q, sc = oracle.quant_per_token(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * sc[:, None].astype(np.float64))
    assert np.all(err <= sc[:, None].astype(np.float64) / 2 * (1 + 1e-6))
    assert q.min() >= -127 and q.max() <= 127
    # every row uses the full code range (its peak maps to +-127)
    assert np.all(np.abs(q).max(axis=1) == 127)
    # static scale: out-of-range values saturate at +-127 (never -128)
    qs, sat = oracle.quant_static(f32([[300.0, -300.0, 127.4, -127.6, 0.2]]), np.float32(1.0))
    np.testing.assert_array_equal(qs[0], [127, -127, 127, -127, 0])
    assert sat == 3


def test_effective_levels():
    """[Review] §2.4: a channel with peak m_i in a tensor with peak m gets about
    2^8 m_i/m levels.  Exact count for a densely filled channel:
    2*rne(127 m_i/m) + 1 (the estimate 256 m_i/m counts 2^8 levels where the
    symmetric quantizer has 255)."""
    _, cases = _golden("effective_levels.txt")
    for c in cases:
        mi, m, est = (float(t) for t in c.split(","))
        assert abs(est - 256 * mi / m) < 1e-9
        ch = np.linspace(-mi, mi, 200001, dtype=np.float32)
        x = np.zeros((2, ch.size), np.float32)
        x[0] = ch
        x[1, 0] = m
        scale = np.float32(m) / np.float32(127)
        q, _ = oracle.quant_static(x, scale)
        levels = np.unique(q[0]).size
        assert levels == 2 * round(127 * mi / m) + 1
        # 2*rne(127 r)+1 vs 256 r: rounding adds at most one code per side
        assert abs(levels - est) <= est * 2 / 256 + 2 + 1e-9


# ---- weights: per-output-channel axis -----------------------------------------------

def test_weight_scale_is_per_output_channel():
    rng = np.random.default_rng(21)
    N, K = 6, 256
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    w[2] *= 50.0                      # one loud output row
    s = rng.uniform(0.5, 2.0, K).astype(np.float32)
    wq, sc = oracle.weight_quant(w, s)
    # each row reaches +-127 at its own peak
    assert np.all(np.abs(wq).max(axis=1) == 127)
    ws = w.astype(np.float64) * s.astype(np.float64)
    np.testing.assert_allclose(sc.astype(np.float64) * 127, np.abs(ws).max(axis=1), rtol=1e-6)
    # dequantized weight within half a step of the smoothed weight (P9 on W)
    err = np.abs(ws - wq.astype(np.float64) * sc[:, None])
    assert np.all(err <= sc[:, None] / 2 * (1 + 1e-6) + 1e-9)
    # row sampling returns the same rows
    wq2, sc2 = oracle.weight_quant(w, s, rows=[4, 2])
    np.testing.assert_array_equal(wq2, wq[[4, 2]])
    np.testing.assert_array_equal(sc2, sc[[4, 2]])


def test_per_input_column_scale_is_rejected():
    """The edge listing takes its weight maxima per input column but applies
    the scale per output column in the GEMM; that cannot be factored out of
    the contraction.  Our per-output-channel quantization reproduces Y, the
    per-input reading applied per output does not (smoothed weights: the
    outlier input channels carry much larger column peaks)."""
    spec = datagen.workload(1).layers[0]
    xc, x, w = datagen.calibration_x(spec), datagen.eval_x(spec), datagen.weights(spec)
    s = oracle.calibrate(xc, w, spec.alpha)["s"]
    y64 = oracle.ref_linear_f64(x, w)
    xq, xs, _ = oracle.smooth_quantize_act(x, s=s)
    wq, ws = oracle.weight_quant(w, s)
    y_ok = oracle.gemm_w8a8(xq, xs, wq, ws)
    wq_bad, cs = oracle.weight_quant_per_input(w, s)
    y_bad = oracle.gemm_w8a8(xq, xs, wq_bad, cs[: spec.N])  # listing's indexing
    rel = lambda y: np.linalg.norm(y - y64) / np.linalg.norm(y64)  # noqa: E731
    assert rel(y_ok) < 0.05
    assert rel(y_bad) > 5 * rel(y_ok)


# ---- static scale -----------------------------------------------------------------

@pytest.mark.parametrize("alpha", (0.0, 0.5, 0.85))
def test_static_scale_equals_second_pass(alpha):
    spec = datagen.workload(1).layers[0]
    xc = datagen.calibration_x(spec)
    a, wm = oracle.colmax(xc), oracle.colmax(datagen.weights(spec))
    s = oracle.smooth_factor(a, wm, alpha)
    second = np.abs(oracle.act_smooth(xc, s)).max()
    assert oracle.static_scale(a, s) == np.float32(max(second, oracle.FLOOR)) / np.float32(127)


# ---- integer GEMM (brute force) ---------------------------------------------------

def test_all_int8_products():
    v = np.arange(-128, 128, dtype=np.int8)
    acc = oracle.gemm_i32(v[:, None], v[:, None])
    np.testing.assert_array_equal(acc, np.outer(v.astype(np.int64), v.astype(np.int64)))


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 8, 256), (7, 2, 64), (2, 7, 129)])
def test_tiny_gemm_brute_force(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    acc = oracle.gemm_i32(xq, wq)
    for m in range(M):
        for n in range(N):
            t = 0
            for k in range(K):
                t += int(xq[m, k]) * int(wq[n, k])
            assert acc[m, n] == t


def test_gemm_int32_range_limit():
    K = 133144  # 127^2 * K < 2^31
    xq = np.full((1, K), 127, np.int8)
    wq = np.full((2, K), -127, np.int8)
    wq[1] = 127
    acc = oracle.gemm_i32(xq, wq)
    assert acc[0, 0] == -127 * 127 * K and acc[0, 1] == 127 * 127 * K
    with pytest.raises(OverflowError):
        oracle.gemm_i32(np.full((1, K + 1), 127, np.int8), np.full((1, K + 1), 127, np.int8))


def test_dequant_within_two_ulps_of_exact_and_bf16_matches_torch():
    rng = np.random.default_rng(4)
    acc = rng.integers(-2**30, 2**30, size=(5, 9), dtype=np.int64).astype(np.int32)
    xs = rng.uniform(1e-3, 1, 5).astype(np.float32)
    ws = rng.uniform(1e-5, 1e-3, 9).astype(np.float32)
    y = oracle.dequant(acc, xs, ws, per_token=True)
    exact = acc.astype(np.float64) * xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    assert np.all(np.abs(y - exact) <= 2.5 * np.spacing(np.abs(y)))
    yt = oracle.dequant(acc, xs[:1], ws, per_token=False)
    exact_t = acc.astype(np.float64) * float(xs[0]) * ws[None, :].astype(np.float64)
    assert np.all(np.abs(yt - exact_t) <= 2.5 * np.spacing(np.abs(yt)))
    # bf16 rounding vs torch's (nearest-even) conversion, incl. exact ties
    vals = np.concatenate([y.ravel(), f32([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16(vals), ref)



def test_dequant_order_hand_example():
    """tests/golden/dequant_order_example.txt ([Edge] §三: the dequant factor
    dx * dw is formed first, then (float)acc times it).  The hand-worked triple
    separates that order from scaling by dx and then by dw by one ulp; a second
    case pins the round-to-nearest-even int32 -> fp32 conversion."""
    g = _golden_kv("dequant_order_example.txt")
    u = lambda k: np.array([int(g[k][0], 16)], np.uint32).view(np.float32)
    acc = np.array([[int(g["acc"][0])]], np.int32)
    y = oracle.dequant(acc, u("dx_bits"), u("dw_bits"), per_token=True)
    assert int(y.view(np.uint32)[0, 0]) == int(g["y_bits"][0], 16)
    assert int(y.view(np.uint32)[0, 0]) != int(g["y_bits_other_order"][0], 16)
    yt = oracle.dequant(acc, u("dx_bits"), u("dw_bits"), per_token=False, w_per_tensor=True)
    assert int(yt.view(np.uint32)[0, 0]) == int(g["y_bits"][0], 16)
    one = np.ones(1, np.float32)
    y2 = oracle.dequant(np.array([[int(g["acc2"][0]), -int(g["acc2"][0])]], np.int32), one,
                        np.ones(2, np.float32), per_token=True)
    assert y2[0, 0] == np.float32(float(g["y2"][0])) and y2[0, 1] == -np.float32(float(g["y2"][0]))


# ---- LayerNorm mode ---------------------------------------------------------------

def test_canonical_sum_hand_cases():
    _, cases = _golden("canonical_sum_cases.txt")
    assert len(cases) == 5
    for c in cases:
        K, elems, expect = [t.strip() for t in c.split(";")]
        v = np.zeros(int(K), np.float32)
        for e in elems.split():
            i, x = e.split(":")
            v[int(i)] = float(x)
        assert oracle.canonical_sum(v) == np.float32(float(expect)), c


def test_canonical_sum_close_to_exact():
    rng = np.random.default_rng(8)
    for K in (64, 512, 4096, 8192, 12288):
        v = rng.normal(0, 3, K).astype(np.float32)
        exact = math.fsum(v.astype(np.float64))
        bound = K * 2**-24 * np.abs(v.astype(np.float64)).sum()
        assert abs(float(oracle.canonical_sum(v)) - exact) <= bound


def test_layernorm_fold_against_fp64_layernorm():
    """LN with (gamma/s, beta/s) equals LN(x; gamma, beta)/s ([Edge] §二) to
    fp32 accuracy; the fp64 reference is numpy's mean/var, not the oracle."""
    spec = datagen.workload(5).layers[0]
    x = datagen.eval_x(spec, M=32)
    gamma, beta = datagen.ln_params(spec)
    rng = np.random.default_rng(12)
    s = rng.uniform(0.05, 20.0, spec.K).astype(np.float32)
    gs, bs = oracle.ln_fold(gamma, beta, s)
    xh = oracle.act_ln(x, gs, bs, eps=1e-5)
    xf = datagen.bf16_bits_to_f32(x).astype(np.float64)
    mu = xf.mean(axis=1, keepdims=True)
    var = xf.var(axis=1, keepdims=True)
    ref = ((xf - mu) / np.sqrt(var + 1e-5) * gamma + beta) / s
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(xh - ref) <= 4e-6 * scale)
    # rows selection consistent
    np.testing.assert_array_equal(oracle.act_ln(x, gs, bs, rows=[5, 1]), xh[[5, 1]])



def test_ln_f64_closed_forms():
    """The fp64 LayerNorm reference (the denominator of the LayerNorm
    workload's int8-vs-fp64 error, [Edge] §二 LN(x) * gamma + beta) on rows
    whose mean and biased variance are known by construction:
      - a constant row has d = 0, so the output is beta exactly;
      - a row alternating c + a, c - a has mean c and biased variance a^2, so
        channel k gives +-a / sqrt(a^2 + eps) * gamma_k + beta_k (the unbiased
        variance would give a^2 K / (K - 1); a swapped sign or a transposed
        gamma / beta fails the per-channel values).
    The same rows stored as bf16 (values exact in 8 bits) give the same result."""
    K = 8
    rng = np.random.default_rng(21)
    gamma = rng.uniform(0.5, 1.5, K)
    beta = rng.normal(0, 0.3, K)
    eps = 1e-5
    c, a = 3.0, 2.0
    sign = np.array([1.0, -1.0] * (K // 2))
    rows = np.stack([np.full(K, 5.25), c + a * sign]).astype(np.float32)
    out = oracle.ln_f64(rows, gamma, beta, eps)
    assert np.array_equal(out[0], beta)
    want = sign * (a / np.sqrt(a * a + eps)) * gamma + beta
    assert np.allclose(out[1], want, rtol=1e-14, atol=1e-14)
    unbiased = sign * (a / np.sqrt(a * a * K / (K - 1) + eps)) * gamma + beta
    assert not np.allclose(out[1], unbiased, rtol=1e-6, atol=1e-6)
    bits = (rows.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(bits), rows)
    np.testing.assert_array_equal(oracle.ln_f64(bits, gamma, beta, eps), out)


def test_ln_f64_matches_fp32_layernorm_to_its_rounding():
    """The fp32 LayerNorm of the fused kernel's contract (canonical sums, one
    rounding per operation) stays within a few fp32 ulps of the fp64 one on
    the LayerNorm workload's tokens, with gamma and beta unfolded (s = 1)."""
    spec = datagen.workload(5).layers[0]
    x = datagen.eval_x(spec, M=8)
    gamma, beta = datagen.ln_params(spec)
    ref = oracle.ln_f64(x, gamma.astype(np.float64), beta.astype(np.float64), 1e-5)
    got = oracle.act_ln(x, gamma, beta, eps=1e-5)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= 4e-6 * scale)


# ---- whole path: eq. (3) and error bounds -------------------------------------------

def test_fp64_identity_config1():
    spec = datagen.workload(1).layers[0]
    xc, x, w = datagen.calibration_x(spec), datagen.eval_x(spec), datagen.weights(spec)
    cal = oracle.calibrate(xc, w, spec.alpha)
    y = oracle.ref_linear_f64(x, w)
    yh = oracle.ref_smoothed_linear_f64(x, w, cal["s"])
    assert np.linalg.norm(y - yh) / np.linalg.norm(y) <= 1e-12


@pytest.mark.parametrize("s_one", [False, True])
def test_output_error_bound_per_element(s_one):
    """|y - Y64| <= sum_k(|xh_k| dw/2 + |wh_k| dx/2 + dx dw/4) + fp32 epilogue
    rounding (quantizer bound of [Review] §2.2 on both operands)."""
    spec = datagen.workload(1).layers[0]
    xc, x, w = datagen.calibration_x(spec), datagen.eval_x(spec), datagen.weights(spec)
    cal = oracle.calibrate(xc, w, spec.alpha)
    s = np.ones(spec.K, np.float32) if s_one else cal["s"]
    wq, ws = oracle.weight_quant(w, s)
    xq, xs, _ = oracle.smooth_quantize_act(x, s=s)
    y = oracle.gemm_w8a8(xq, xs, wq, ws)
    xh = oracle.as_f64(x) / s.astype(np.float64)
    wh = oracle.as_f64(w) * s.astype(np.float64)
    y64 = xh @ wh.T
    dx = xs.astype(np.float64)[:, None]
    dw = ws.astype(np.float64)[None, :]
    bound = (np.abs(xh).sum(1)[:, None] * dw / 2 + dx * np.abs(wh).sum(1)[None, :] / 2
             + spec.K * dx * dw / 4)
    bound = bound * (1 + 1e-5) + 4 * np.spacing(np.abs(y).astype(np.float32))
    assert np.all(np.abs(y - y64) <= bound)
    if s_one:  # no smoothing: the activation side is the identity
        np.testing.assert_array_equal(oracle.act_smooth(x, s), x)


def test_smoothing_reduces_error_on_outlier_layer():
    """The point of the method: with outlier channels, alpha = 0.5 beats s = 1
    (naive W8A8) on the static per-tensor setting of the single-linear case."""
    spec = datagen.workload(1).layers[0]
    xc, x, w = datagen.calibration_x(spec), datagen.eval_x(spec), datagen.weights(spec)
    y64 = oracle.ref_linear_f64(x, w)

    def run(s):
        a = oracle.colmax(xc)
        st = oracle.static_scale(a, s)
        wq, ws = oracle.weight_quant(w, s)
        xq, xs, _ = oracle.smooth_quantize_act(x, s=s, static=st)
        y = oracle.gemm_w8a8(xq, xs, wq, ws, per_token=False)
        return np.linalg.norm(y - y64) / np.linalg.norm(y64)

    cal = oracle.calibrate(xc, w, 0.5)
    e_sq = run(cal["s"])
    e_naive = run(np.ones(spec.K, np.float32))
    assert e_sq < 0.5 * e_naive


# ---- per-tensor settings SmoothQuant-O1/O2/O3 ([Review] §6.3) ----------------------

def _golden_kv(name):
    kv = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.split()
    return kv


def _bits(x):
    return int(np.array(np.float32(x)).view(np.uint32))


def test_per_tensor_hand_example():
    """tests/golden/per_tensor_example.txt: the weight step, the dynamic
    activation step and every code, worked by hand (one exact tie included)."""
    g = _golden_kv("per_tensor_example.txt")
    w = np.array(g["w"], np.float32).reshape([int(v) for v in g["w_shape"]])
    wq, dw = oracle.weight_quant_per_tensor(w, np.ones(w.shape[1], np.float32))
    assert _bits(dw[0]) == int(g["w_step_bits"][0], 16)
    assert wq.ravel().tolist() == [int(v) for v in g["w_codes"]]
    _, row_steps = oracle.weight_quant(w, np.ones(w.shape[1], np.float32))
    assert [_bits(v) for v in row_steps] == [int(v, 16) for v in g["w_row_step_bits"]]
    x = np.array(g["x"], np.float32).reshape([int(v) for v in g["x_shape"]])
    xq, dx = oracle.quant_dynamic_per_tensor(x)
    assert _bits(dx[0]) == int(g["x_step_bits"][0], 16)
    assert xq.ravel().tolist() == [int(v) for v in g["x_codes"]]
    _, tok_steps = oracle.quant_per_token(x)
    assert [_bits(v) for v in tok_steps] == [int(v, 16) for v in g["x_row_step_bits"]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_per_tensor_weight_step_from_column_maxima(seed):
    """Invariant of the per-tensor weight step ([Review] §6.3): rounding and a
    multiplication by s_k > 0 are monotone, so max over n, k of |RN(W[n,k] s_k)|
    equals max_k RN(max_n |W[n,k]| s_k); the step is RN(max(FLOOR, that) / 127).
    Checked on bf16 weights with outlier and all-zero columns and s spread over
    six decades, the step computed from the column maxima in numpy fp32."""
    rng = np.random.default_rng(500 + seed)
    N, K = 96, 320
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    w[:, rng.choice(K, 4, replace=False)] *= 300.0
    w[:, rng.choice(K, 3, replace=False)] = 0.0
    w = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(w))
    s = (10.0 ** rng.uniform(-3, 3, K)).astype(np.float32)
    _, dw = oracle.weight_quant_per_tensor(w, s)
    colmax = np.abs(w).max(axis=0).astype(np.float32)
    m = np.max(colmax * s)  # fp32 products, each rounded once
    step = np.float32(max(np.float32(1e-7), m)) / np.float32(127.0)
    assert _bits(dw[0]) == _bits(step)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_per_tensor_step_is_max_of_finer_steps(seed):
    """step = RN(max(FLOOR, m)/127) is monotone in m, so the per-tensor weight
    step equals the largest per-output-channel step and the dynamic per-tensor
    activation step the largest per-token step, bit for bit; rows that attain
    the maximum get identical codes under both granularities, and every other
    row uses at most as many levels."""
    rng = np.random.default_rng(seed)
    N, K = 37, 96
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[5, 7] = 0.9
    s = rng.uniform(0.2, 5.0, K).astype(np.float32)
    wq_t, dw = oracle.weight_quant_per_tensor(w, s)
    wq_c, dwn = oracle.weight_quant(w, s)
    assert dw[0] == dwn.max()
    top = np.flatnonzero(dwn == dw[0])
    assert np.array_equal(wq_t[top], wq_c[top])
    assert np.all(np.abs(wq_t).max(axis=1) <= np.abs(wq_c).max(axis=1))
    xh = (rng.standard_normal((29, K)) * 3).astype(np.float32)
    xh[11, 3] = -60.0
    q_t, d = oracle.quant_dynamic_per_tensor(xh)
    q_c, dt = oracle.quant_per_token(xh)
    assert d[0] == dt.max()
    top = np.flatnonzero(dt == d[0])
    assert np.array_equal(q_t[top], q_c[top])


def test_dynamic_per_tensor_error_bound():
    """The symmetric quantizer's bound |x - q d| <= d/2 holds for every element
    (a dynamic step never clamps), and the batch maximum maps to +-127."""
    rng = np.random.default_rng(3)
    xh = (rng.standard_normal((64, 128)) * 2).astype(np.float32)
    q, d = oracle.quant_dynamic_per_tensor(xh)
    err = np.abs(xh.astype(np.float64) - q.astype(np.float64) * np.float64(d[0]))
    assert err.max() <= np.float64(d[0]) / 2 * (1 + 2.0 ** -20)
    assert int(np.abs(q).max()) == 127


def test_dequant_per_tensor_weight_is_broadcast():
    """A per-tensor weight step dequantizes exactly like a per-channel vector
    filled with that step."""
    rng = np.random.default_rng(4)
    acc = rng.integers(-2 ** 30, 2 ** 30, size=(7, 13), dtype=np.int64).astype(np.int32)
    xs = rng.uniform(1e-3, 1e-1, 7).astype(np.float32)
    d = np.float32(0.0123)
    y_t = oracle.dequant(acc, xs, np.array([d], np.float32), per_token=True, w_per_tensor=True)
    y_c = oracle.dequant(acc, xs, np.full(13, d, np.float32), per_token=True)
    assert np.array_equal(y_t.view(np.uint32), y_c.view(np.uint32))


# ---- fused epilogue: bias, ReLU, requantization for the next linear ---------------

def test_fused_epilogue_hand_example():
    g = _golden_kv("fused_epilogue_example.txt")
    f = lambda k: np.array(g[k], np.float32)
    out = oracle.epilogue(f("y")[None, :], f("bias"), relu=True)
    assert np.array_equal(out[0], f("after_relu"))
    q, sat = oracle.requant(out, f("next_s"), np.float32(g["step"][0]))
    assert q[0].tolist() == [int(v) for v in g["codes"]]
    assert sat == int(g["saturated"][0])


def test_requant_reduces_to_the_pinned_act_path():
    """Requantizing fp32 outputs equals the (separately pinned) plain smoothing
    followed by the static quantizer on the same fp32 tensor -- the fused and
    the unfused graph give the same codes -- and with s' = 1 it is the static
    quantizer itself."""
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((23, 192)) * 4).astype(np.float32)
    y[3, 5] = 900.0                                    # saturates
    ns = rng.uniform(0.05, 20.0, 192).astype(np.float32)
    D = np.float32(0.031)
    q, sat = oracle.requant(y, ns, D)
    xh = oracle.act_smooth(y, ns)
    q2, sat2 = oracle.quant_static(xh, D)
    assert np.array_equal(q, q2) and sat == sat2 and sat >= 1
    q1, _ = oracle.requant(y, None, D)
    q3, _ = oracle.quant_static(y, D)
    assert np.array_equal(q1, q3)


def test_epilogue_identities_and_relu_sign():
    """No bias and no ReLU is the identity; ReLU outputs are >= +0 (no -0) and
    equal the input where it is positive; a zero bias changes nothing."""
    rng = np.random.default_rng(6)
    y = (rng.standard_normal((9, 40)) * 3).astype(np.float32)
    y[0, :4] = [-0.0, 0.0, -1e-30, 1e-30]
    assert np.array_equal(oracle.epilogue(y).view(np.uint32), y.view(np.uint32))
    r = oracle.epilogue(y, relu=True)
    assert np.all(np.signbit(r) == False)              # noqa: E712
    pos = y > 0
    assert np.array_equal(r[pos], y[pos]) and np.all(r[~pos] == 0)
    z = oracle.epilogue(y, np.zeros(40, np.float32))
    nz = y != 0                                        # -0 + +0 is +0 under RN
    assert np.array_equal(z[nz].view(np.uint32), y[nz].view(np.uint32))


# ---- int8 attention products ([Review] §5.6, Fig. 6) ------------------------------

def test_int8_attention_scores_within_quantizer_bound():
    """S = Q K^T with both operands quantized per token (no smoothing): every
    dequantized score lies within the quantizer's error bound of the fp64
    product, sum_k(|q_k| dk/2 + |k_k| dq/2 + dq dk/4) plus fp32 rounding, and
    the batched oracle is the per-head GEMM with the head's scales."""
    rng = np.random.default_rng(11)
    H, S, d = 3, 37, 64
    q = rng.standard_normal((H, S, d)).astype(np.float32)
    k = rng.standard_normal((H, S, d)).astype(np.float32)
    q[1, 4, 9] = 30.0                                  # a head with an outlier query
    ones = np.ones(d, np.float32)
    qq, qs = zip(*[oracle.quant_per_token(oracle.act_smooth(q[h], ones)) for h in range(H)])
    kq, ks = zip(*[oracle.quant_per_token(oracle.act_smooth(k[h], ones)) for h in range(H)])
    qq, qs, kq, ks = map(np.stack, (qq, qs, kq, ks))
    s = oracle.bmm_w8a8(qq, qs, kq, ks)
    for h in range(H):
        exact = q[h].astype(np.float64) @ k[h].astype(np.float64).T
        dq, dk = qs[h].astype(np.float64)[:, None], ks[h].astype(np.float64)[None, :]
        bound = (np.abs(q[h]).astype(np.float64) @ np.ones((d, 1))) * dk / 2 \
            + dq / 2 * (np.ones((1, d)) @ np.abs(k[h]).astype(np.float64).T) + d * dq * dk / 4
        err = np.abs(s[h].astype(np.float64) - exact)
        assert np.all(err <= bound * (1 + 1e-6) + np.abs(exact) * 2.0 ** -22)
        assert np.array_equal(s[h], oracle.gemm_w8a8(qq[h], qs[h], kq[h], ks[h]))


# ---- robust calibration ([Teach] §四, §六, §八) ------------------------------------

def test_channel_quantile_is_the_inverted_cdf_quantile():
    """Nearest rank equals numpy's inverted-CDF quantile (smallest value whose
    empirical CDF reaches q) column by column.  q T is kept clear of integers
    (the two rules may round such a product differently; the exact-integer
    case is pinned in test_channel_quantile_extremes)."""
    rng = np.random.default_rng(21)
    for T in (1, 37, 513, 1001):
        x = rng.standard_normal((T, 48)).astype(np.float32)
        for q in (0.25, 0.5, 0.9, 0.999, 1.0):
            qd = float(np.float32(q))
            ref = np.quantile(np.abs(x), qd, axis=0, method="inverted_cdf")
            got = oracle.channel_quantile(x, q)
            assert np.array_equal(got, np.maximum(ref, oracle.FLOOR).astype(np.float32)), (T, q)


def test_channel_quantile_order_statistic_with_ties():
    """For rank r: fewer than r magnitudes lie below the result and at least r at
    or below it (integer data with many ties; bf16 input bits)."""
    import datagen
    rng = np.random.default_rng(22)
    x = rng.integers(-6, 7, size=(301, 40)).astype(np.float32)
    xb = datagen.f32_to_bf16_bits(x)
    for q in (0.01, 0.3, 0.5, 0.77, 1.0):
        v = oracle.channel_quantile(xb, q)
        r = oracle.quantile_rank(301, q)
        a = np.abs(x)
        below = (a < v[None, :]).sum(axis=0)
        at_or_below = (a <= v[None, :]).sum(axis=0)
        zero_col = v == oracle.FLOOR                   # a zero quantile is floored
        assert np.all(below[~zero_col] < r) and np.all(at_or_below >= r)


def test_channel_quantile_extremes():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    assert np.array_equal(oracle.channel_quantile(x, 1.0), oracle.colmax(x))   # the peak (a1)
    mn = np.maximum(np.abs(x).min(axis=0), oracle.FLOOR)
    assert np.array_equal(oracle.channel_quantile(x, 1e-9), mn)                  # rank 1
    assert oracle.quantile_rank(64, 1e-9) == 1 and oracle.quantile_rank(64, 1.0) == 64
    assert oracle.quantile_rank(10, 0.35) == 4 and oracle.quantile_rank(8, 0.5) == 4
    assert np.all(oracle.channel_quantile(np.empty((0, 8), np.float32), 0.5) == oracle.FLOOR)


def test_calibrate_from_peak_statistic_is_calibrate():
    """A given statistic equal to the calibration peak reproduces the offline
    half bit for bit, LayerNorm fold included; a lower robust statistic lowers
    the static step, which then saturates the tokens above it."""
    rng = np.random.default_rng(24)
    xc = rng.standard_normal((128, 64)).astype(np.float32)
    xc[:, 5] *= 40.0
    w = (rng.standard_normal((48, 64)) * 0.05).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    b = (rng.standard_normal(64) * 0.1).astype(np.float32)
    ref = oracle.calibrate(xc, w, 0.5, g, b)
    got = oracle.calibrate(None, w, 0.5, g, b, act_stat=oracle.colmax(xc))
    for k in ("a", "wmax", "s", "wq", "w_scale", "static_scale", "g_s", "b_s"):
        assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), k
    rob = oracle.calibrate(None, w, 0.5, act_stat=oracle.channel_quantile(xc, 0.9))
    assert rob["static_scale"] < ref["static_scale"]
    xh = oracle.act_smooth(xc, rob["s"])
    assert oracle.clip_counts(xh, rob["static_scale"])[0] > 0
    xh0 = oracle.act_smooth(xc, ref["s"])
    assert oracle.clip_counts(xh0, ref["static_scale"])[0] == 0      # the peak never clips


def test_clip_counts_hand_example():
    """Step 0.5 (x / step exact): 63.7 -> 127.4 -> 127 kept; 63.75 -> 127.5 -> 128
    (tie to even) clipped; 63.25 -> 126.5 -> 126 kept; -63.75 clipped; 150 and
    -64 clipped; 0 kept."""
    xh = np.array([[63.7, 63.75, 63.25, -63.75],
                   [150.0, -64.0, 0.0, 1.0]], np.float32)
    total, per = oracle.clip_counts(xh, 0.5)
    assert total == 4 and per.tolist() == [1, 2, 0, 1]
    assert oracle.quant_static(xh, 0.5)[1] == total          # the C quantizer's own count


def test_alpha_search_lossless_construction():
    """Integer data whose column peaks m_j are the same for X and W (so s = 1
    exactly at alpha = 0.5 and nowhere else) and whose every row attains 127:
    at alpha = 0.5 every step is exactly 1 and the quantized linear is exact
    (err = werr = 0), so 0.5 is chosen; other alphas smooth unevenly and lose."""
    rng = np.random.default_rng(25)
    T, K, N = 6, 16, 10
    m = np.concatenate([np.full(4, 127), rng.integers(20, 127, size=K - 4)])
    def grid(R):
        a = np.stack([rng.integers(-mj, mj + 1, size=R) for mj in m], axis=1).astype(np.float32)
        for j in range(K):
            a[j % R, j] = m[j] if j % 2 else -m[j]          # each column attains m_j
        for r in range(R):
            a[r, r % 4] = 127.0                              # each row attains 127
        return a
    x, w = grid(T), grid(N)
    assert np.array_equal(oracle.colmax(x), oracle.colmax(w))
    alphas = [0.25, 0.5, 0.75]
    for mode in ("per_token", "static", "dynamic_per_tensor"):
        for wpt in (False, True):
            err, werr, best = oracle.alpha_search(x, w, alphas, mode=mode, w_per_tensor=wpt)
            assert err[1] == 0.0 and werr[1] == 0.0 and best == 1, (mode, wpt)
            assert err[0] > 0 and err[2] > 0


def test_alpha_search_hand_example():
    """One token x = (1, 100), one output w = (1, 1), alpha = 0.5: s = (1, 10),
    smoothed x and w both (1, 10), steps 10/127, codes (13, 127) on both sides,
    y_q = 16298 * (10/127)^2 against y = 101; the weight error is
    (1 - 13*10/127)^2 / (1 + 100).  Exact rationals; the fp32 steps and product
    (about 3 ulp on y_q, i.e. 101 * 1.8e-7 against a difference of 0.048) move
    err by at most 8e-4 relative, werr by far less."""
    from fractions import Fraction as F
    x = np.array([[1.0, 100.0]], np.float32)
    w = np.array([[1.0, 1.0]], np.float32)
    cal = oracle.calibrate(x, w, 0.5)
    assert cal["s"].tolist() == [1.0, 10.0]
    assert oracle.smooth_quantize_act(x, s=cal["s"])[0].tolist() == [[13, 127]]
    assert cal["wq"].tolist() == [[13, 127]]
    err, werr, best = oracle.alpha_search(x, w, [0.5])
    d = F(10, 127)
    e_exact = (F(16298) * d * d - 101) ** 2 / F(101) ** 2
    w_exact = (1 - 13 * d) ** 2 / F(101)
    assert abs(err[0] / float(e_exact) - 1) < 1e-3
    assert abs(werr[0] / float(w_exact) - 1) < 1e-4 and best == 0


def test_alpha_search_power_of_two_invariance():
    """At alpha = 1 (s = a) and alpha = 0 (s = 1/w) doubling W scales every
    intermediate by an exact power of two: both errors are unchanged bit for
    bit, in every activation mode."""
    rng = np.random.default_rng(26)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    x[:, 3] *= 30.0
    w = (rng.standard_normal((24, 64)) * 0.02).astype(np.float32)
    for mode in ("per_token", "static", "dynamic_per_tensor"):
        e1, w1, _ = oracle.alpha_search(x, w, [0.0, 1.0], mode=mode)
        e2, w2, _ = oracle.alpha_search(x, 2 * w, [0.0, 1.0], mode=mode)
        assert np.array_equal(e1, e2) and np.array_equal(w1, w2), mode
