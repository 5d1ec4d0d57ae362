"""GPU parity of the robust-calibration calls ([Teach] §四: a robust
per-channel statistic instead of the peak, alpha searched with the weight
range; §六: the clip rate per layer; §八: candidate alphas compared on
saturation and weight quantization error) against the oracle:
  * sq_channel_quantile bit for bit (bf16 and fp32, ties, every rank), on the
    65536-token calibration set of the LayerNorm workload on sampled channels;
  * sq_calibrate_stat bit for bit (LayerNorm fold, per-tensor weight step);
  * sq_clip_count exactly (total and per channel) through every quantizer
    kernel (short rows, cached rows, uncached rows, long rows, LayerNorm);
  * sq_alpha_search within 1e-9 relative (fp64 sums in another order) with the
    same chosen alpha.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, c5_inputs, dev, sample_idx, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _data(T, K, seed, dtype, ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        x = rng.integers(-9, 10, size=(T, K)).astype(np.float32)
    else:
        x = rng.standard_normal((T, K)).astype(np.float32)
        x[:, rng.choice(K, size=max(1, K // 50), replace=False)] *= 40.0
    return datagen.f32_to_bf16_bits(x) if dtype == "bf16" else x


QCASES = [
    # T, K, dtype, ties
    (1, 64, "bf16", False),
    (37, 320, "f32", False),
    (513, 4096, "bf16", False),
    (1000, 192, "f32", True),
    (2048, 1024, "bf16", True),
    (300, 64, "f32", False),
]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: f"T{c[0]}_K{c[1]}_{c[2]}" + ("_ties" if c[3] else ""))
def test_channel_quantile_every_channel(case):
    T, K, dt, ties = case
    x = _data(T, K, T + K, dt, ties)
    xt = to_dev(x, dev())
    for q in (1.0, 0.999, 0.9, 0.5, 0.01, 1e-9):
        say(f"[case] quantile T={T} K={K} {dt} q={q}")
        got = to_np(sq.sq_channel_quantile(xt, q))
        assert_same(f"quantile q={q}", got, oracle.channel_quantile(x, q))


def test_channel_quantile_empty_and_peak():
    d = dev()
    out = sq.sq_channel_quantile(torch.empty((0, 128), dtype=torch.bfloat16, device=d), 0.5)
    assert np.all(to_np(out) == oracle.FLOOR)
    x = _data(777, 512, 5, "bf16")
    cal = sq.sq_calibrate(to_dev(x, d), to_dev(_data(64, 512, 6, "bf16"), d), 0.5)
    assert_same("q=1 is the peak", to_np(sq.sq_channel_quantile(to_dev(x, d), 1.0)),
                to_np(cal["x_absmax"]))


def test_channel_quantile_ln8192_calibration_sampled():
    """The 65536 x 8192 bf16 calibration set (1 GiB): every channel computed,
    32 sampled channels checked against the oracle."""
    c5 = c5_inputs()
    xt = to_dev(c5["xc"], dev())
    cols = sample_idx(c5["xc"].shape[1], 32, 55)
    sub = np.ascontiguousarray(c5["xc"][:, cols])
    for q in (0.9999, 0.99, 0.5):
        say(f"[case] quantile ln8192 q={q}")
        got = to_np(sq.sq_channel_quantile(xt, q))
        assert_same(f"ln8192 quantile q={q}", got[cols], oracle.channel_quantile(sub, q))
        assert np.all(got <= to_np(sq.sq_channel_quantile(xt, 1.0)))


@pytest.mark.parametrize("wmode", ["per_channel", "per_tensor"])
@pytest.mark.parametrize("ln", [False, True])
def test_calibrate_stat_matches_oracle(ln, wmode):
    d = dev()
    rng = np.random.default_rng(7)
    K, N = 512, 300
    xc = _data(256, K, 8, "bf16")
    w = datagen.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    g = rng.uniform(0.5, 1.5, K).astype(np.float32) if ln else None
    b = (rng.standard_normal(K) * 0.1).astype(np.float32) if ln else None
    stat = sq.sq_channel_quantile(to_dev(xc, d), 0.99)
    say(f"[case] calibrate_stat ln={ln} {wmode}")
    got = sq.sq_calibrate_stat(stat, to_dev(w, d), 0.5, None if g is None else to_dev(g, d),
                               None if b is None else to_dev(b, d), w_mode=wmode)
    ref = oracle.calibrate(None, w, 0.5, g, b, act_stat=oracle.channel_quantile(xc, 0.99),
                           w_per_tensor=wmode == "per_tensor")
    assert_same("a", to_np(got["a"]), ref["a"])
    for k in ("s", "wq", "w_scale"):
        assert_same(k, to_np(got[k]), ref[k])
    assert_same("static", to_np(got["static_scale"])[0], ref["static_scale"])
    if ln:
        assert_same("g_s", to_np(got["ln_gamma_s"]), ref["g_s"])
        assert_same("b_s", to_np(got["ln_beta_s"]), ref["b_s"])


CLIP = [
    # M, K, dtype, ln: short rows, cached rows, uncached rows (4 and 8 chunks per lane),
    # long rows, LayerNorm
    (300, 128, "bf16", False),
    (97, 4096, "f32", False),
    (17, 24576, "bf16", False),
    (9, 40960, "f32", False),
    (33, 65536, "bf16", False),
    (64, 8192, "bf16", True),
    (5, 24576, "f32", True),
]


@pytest.mark.parametrize("case", CLIP, ids=lambda c: f"M{c[0]}_K{c[1]}_{c[2]}" + ("_ln" if c[3] else ""))
def test_clip_count_exact(case):
    """A static step from a low quantile of the same tokens saturates many
    elements; total and per-channel counts equal the oracle's exactly."""
    M, K, dt, ln = case
    d = dev()
    rng = np.random.default_rng(M + K)
    x = _data(M, K, M * 3 + K, dt)
    if ln:
        g = rng.uniform(0.5, 1.5, K).astype(np.float32)
        b = (rng.standard_normal(K) * 0.1).astype(np.float32)
        s = (rng.uniform(0.5, 2.0, K)).astype(np.float32)
        gs, bs = oracle.ln_fold(g, b, s)
        xh = oracle.act_ln(x, gs, bs)
    else:
        s = (rng.uniform(0.5, 2.0, K)).astype(np.float32)
        xh = oracle.act_smooth(x, s)
    # step of the 0.9-quantile of |xh| over the whole tensor: about 10% clip
    step = np.float32(np.quantile(np.abs(xh), 0.9) / 127.0)
    tot, per = oracle.clip_counts(xh, step)
    assert tot > 0
    st = torch.tensor([step], dtype=torch.float32, device=d)
    say(f"[case] clip M={M} K={K} {dt} ln={ln}")
    if ln:
        cnt, pc = sq.sq_clip_count(to_dev(x, d), st, ln_gamma_s=to_dev(gs, d),
                                   ln_beta_s=to_dev(bs, d), per_channel=True)
    else:
        cnt, pc = sq.sq_clip_count(to_dev(x, d), st, s=to_dev(s, d), per_channel=True)
    assert int(cnt.item()) == tot
    assert np.array_equal(to_np(pc).astype(np.int64), per)
    cnt2, none = sq.sq_clip_count(to_dev(x, d), st, s=None if ln else to_dev(s, d),
                                  ln_gamma_s=to_dev(gs, d) if ln else None,
                                  ln_beta_s=to_dev(bs, d) if ln else None)
    assert none is None and int(cnt2.item()) == tot


def test_clip_count_peak_calibration_never_clips():
    """r11: the static step from the calibration peaks never saturates the
    calibration tokens; a 0.9-quantile statistic does."""
    d = dev()
    rng = np.random.default_rng(3)
    xc = _data(512, 1024, 9, "bf16")
    w = datagen.f32_to_bf16_bits((rng.standard_normal((256, 1024)) * 0.02).astype(np.float32))
    xt = to_dev(xc, d)
    cal = sq.sq_calibrate(xt, to_dev(w, d), 0.5)
    cnt, _ = sq.sq_clip_count(xt, cal["static_scale"], s=cal["s"])
    assert int(cnt.item()) == 0
    rob = sq.sq_calibrate_stat(sq.sq_channel_quantile(xt, 0.9), to_dev(w, d), 0.5)
    cnt, _ = sq.sq_clip_count(xt, rob["static_scale"], s=rob["s"])
    ref = oracle.calibrate(None, w, 0.5, act_stat=oracle.channel_quantile(xc, 0.9))
    assert int(cnt.item()) == oracle.clip_counts(oracle.act_smooth(xc, ref["s"]),
                                                 ref["static_scale"])[0] > 0


ACASES = [
    # T, N, K, x dtype, w dtype, mode, w mode
    (64, 96, 256, "bf16", "bf16", "per_token", "per_channel"),
    (100, 130, 512, "f32", "bf16", "static", "per_channel"),
    (33, 200, 128, "bf16", "f32", "dynamic_per_tensor", "per_tensor"),
    (257, 64, 1024, "bf16", "bf16", "per_token", "per_tensor"),
]
ALPHAS = [0.0, 0.25, 0.5, 0.75, 0.85, 1.0]


def _rel_close(a, b, tol=1e-9):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= tol * np.maximum(np.abs(b), 1e-300))


@pytest.mark.parametrize("case", ACASES, ids=lambda c: f"T{c[0]}_N{c[1]}_K{c[2]}_{c[5]}_{c[6]}")
def test_alpha_search_matches_oracle(case):
    T, N, K, xdt, wdt, mode, wmode = case
    d = dev()
    rng = np.random.default_rng(T + N + K)
    xc = _data(T, K, T * 5 + K, xdt)
    wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w = datagen.f32_to_bf16_bits(wf) if wdt == "bf16" else wf
    say(f"[case] alpha search T={T} N={N} K={K} {mode} {wmode}")
    err, werr, best = sq.sq_alpha_search(to_dev(xc, d), to_dev(w, d), ALPHAS, mode=mode,
                                         w_mode=wmode)
    e_ref, w_ref, b_ref = oracle.alpha_search(xc, w, ALPHAS, mode=mode,
                                              w_per_tensor=wmode == "per_tensor")
    assert _rel_close(to_np(err), e_ref), (to_np(err), e_ref)
    assert _rel_close(to_np(werr), w_ref), (to_np(werr), w_ref)
    gb = int(best.item())
    assert gb == b_ref or abs(e_ref[gb] - e_ref[b_ref]) <= 1e-9 * e_ref[b_ref]


def test_alpha_search_opt67b_qkv():
    """The qkv linear of the OPT-6.7B workload (512 calibration tokens, 4096 ->
    12288) at three alphas; the oracle's fp64 product and int8 GEMMs run in full."""
    spec = datagen.workload(2).layers[0]
    xc, w = datagen.calibration_x(spec), datagen.weights(spec)
    d = dev()
    al = [0.25, 0.5, 0.75]
    say("[case] alpha search opt6.7b qkv")
    err, werr, best = sq.sq_alpha_search(to_dev(xc, d), to_dev(w, d), al)
    e_ref, w_ref, b_ref = oracle.alpha_search(xc, w, al)
    assert _rel_close(to_np(err), e_ref) and _rel_close(to_np(werr), w_ref)
    assert int(best.item()) == b_ref
