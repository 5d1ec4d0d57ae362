"""Quantizer steps at the ends of their finite range, every element against
the oracle.

The per-token step is d = RN(max(FLOOR, m) / 127) of the row maximum m
([Review] §2.2; FLOOR = 1e-7 is reading r6), and the codes are rne(x / d).
The kernels form d and RN(1/d) without the IEEE division sequences (a
correctly rounded quotient by 127 from RN(1/127), then the two-fma
reciprocal), which is exact only while d stays inside the reciprocal's
range; these rows put m at both ends of the finite range:

  all zeros and maxima below the floor (step FLOOR / 127), a maximum just
  above the floor, maxima near the largest bf16 and fp32 values (d near
  2.7e36, RN(1/d) near 3.7e-37), a power-of-two step 2^120, and ordinary rows
  between them (odd row counts, so the two-row kernels also see a lone last
  row).

Row lengths select every per-token kernel (rows packed in a wave, one row per
block with cached factors, the two-row kernels with one and two chunks per
lane, the long-row kernel at four and six chunks per lane, the multi-sweep
kernel), bf16 and fp32 inputs, the LayerNorm kernels (two-row, one-row and
cached) with folded gamma' / beta' that scale every normalized row far up or
down, the dynamic per-tensor step, and the weight quantizer's row kernels
(sq_calibrate at alpha = 1 with s = 1, so the weight rows carry the same
maxima; per-channel and per-tensor steps).  Codes and steps must match bit
for bit.  NaN and Inf inputs are outside the contract and are not used.
"""
import numpy as np
import pytest

import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

BF16_MAX = np.float32(3.3895313892515355e38)  # largest finite bf16
F32_MAX = np.finfo(np.float32).max


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, rounded to nearest even (finite
    inputs stay finite: every value here is at most BF16_MAX in magnitude)."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def extreme_rows(rng, K, xdt):
    """Nine rows of K values whose maxima span the finite range."""
    top = BF16_MAX if xdt == "bf16" else F32_MAX
    rows = np.zeros((9, K), np.float32)
    u = lambda lo, hi: rng.uniform(lo, hi, K).astype(np.float32) * rng.choice([-1.0, 1.0], K)
    # 0: all zeros
    rows[1] = u(0.0, 3e-8)                          # maximum below the floor
    rows[2] = u(0.0, 1.2e-7)                        # maximum just above the floor
    rows[2, rng.integers(K)] = 1.5e-7
    rows[3] = u(1e37, 3.0e38)                       # near the largest value
    rows[3, rng.integers(K)] = top
    rows[4] = rng.standard_normal(K).astype(np.float32)
    rows[5] = u(0.0, 1.0) * np.float32(3.0e38)
    rows[5, rng.integers(K)] = -top                 # the largest magnitude, negative
    rows[6, rng.integers(K)] = 1e-30                # one tiny element, the rest zero
    rows[7] = u(0.0, 1.0) * np.float32(127.0 * 2.0 ** 120)
    rows[7, rng.integers(K)] = np.float32(127.0 * 2.0 ** 120)   # step exactly 2^120
    rows[8] = u(1e19, 1e21)
    if xdt == "bf16":
        return to_bf16_bits(rows)
    return rows


# row lengths: 128 (rows packed in a wave), 512 (one row per block, cached
# factors), 2048 / 4096 (two-row kernel, one chunk per lane: 256 / 512 lanes),
# 16384 (two-row kernel, two chunks per lane), 24576 / 49152 (long-row kernel,
# four / six chunks per lane), 65536 (multi-sweep kernel)
PLAIN_K = [128, 512, 2048, 4096, 16384, 24576, 49152, 65536]


@pytest.mark.parametrize("K", PLAIN_K)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_per_token_step_extremes(K, xdt):
    d = dev()
    rng = np.random.default_rng(K * 3 + (1 if xdt == "f32" else 0))
    x = extreme_rows(rng, K, xdt)
    # factors 1, 2 and 4: x / s stays exact and finite at both ends
    s = (2.0 ** rng.integers(0, 3, K)).astype(np.float32)
    say(f"[case] per-token step extremes K={K} x={xdt}")
    xq, xs = sq.sq_smooth_quantize_act(to_dev(x, d), to_dev(s, d), mode="per_token")
    q_o, s_o, _ = oracle.smooth_quantize_act(x, s=s)
    assert_same("x_scale", to_np(xs), s_o)
    assert_same("xq", to_np(xq), q_o)
    # the steps really reach both ends
    assert s_o[0] == np.float32(1e-7) / np.float32(127)
    assert s_o[1] == s_o[0] and s_o[6] == s_o[0]
    assert s_o[3] > np.float32(1e35) and s_o[5] > np.float32(1e35)


@pytest.mark.parametrize("K", [512, 4096, 49152])
def test_dynamic_per_tensor_step_extremes(K):
    d = dev()
    rng = np.random.default_rng(K + 11)
    x = extreme_rows(rng, K, "bf16")
    s = (2.0 ** rng.integers(0, 3, K)).astype(np.float32)
    say(f"[case] dynamic per-tensor step extremes K={K}")
    xq, xs = sq.sq_smooth_quantize_act(to_dev(x, d), to_dev(s, d), mode="dynamic_per_tensor")
    q_o, s_o, _ = oracle.smooth_quantize_act(x, s=s, dynamic_per_tensor=True)
    assert_same("x_scale", to_np(xs), s_o)
    assert_same("xq", to_np(xq), q_o)
    # rows of zeros and tiny values quantize to 0 under the batch's huge step
    assert not np.any(to_np(xq)[[0, 1, 2, 6]])


# LayerNorm row lengths: 2048 / 4096 / 8192 (two-row kernel, one to four chunks
# per lane), 12288 (one-row kernel), 24576 (uncached rows)
LN_K = [2048, 4096, 8192, 12288, 24576]


@pytest.mark.parametrize("K", LN_K)
@pytest.mark.parametrize("scale", [1e36, 1e-30])
def test_layernorm_step_extremes(K, scale):
    """gamma' = scale * U(0.5, 1), beta' = 0: every normalized row is scaled
    near the top of the range (|LN(x)| <= sqrt(K)) or below the floor; a
    constant row normalizes to zeros (step FLOOR / 127)."""
    d = dev()
    rng = np.random.default_rng(K + int(scale > 1))
    M = 7
    x = rng.standard_normal((M, K)).astype(np.float32) * 3.0
    x[2] = 1.5                                       # constant row
    x[4, rng.integers(K)] = 200.0                    # one outlier
    xb = to_bf16_bits(x)
    g = (rng.uniform(0.5, 1.0, K) * scale).astype(np.float32)
    b = np.zeros(K, np.float32)
    say(f"[case] LayerNorm step extremes K={K} gamma' ~ {scale:g}")
    xq, xs = sq.sq_smooth_quantize_act(to_dev(xb, d), None, mode="per_token",
                                       ln_gamma_s=to_dev(g, d), ln_beta_s=to_dev(b, d))
    q_o, s_o, _ = oracle.smooth_quantize_act(xb, g_s=g, b_s=b)
    assert_same("x_scale", to_np(xs), s_o)
    assert_same("xq", to_np(xq), q_o)
    floor_step = np.float32(1e-7) / np.float32(127)
    assert s_o[2] == floor_step
    if scale > 1:
        assert np.all(np.delete(s_o, 2) > np.float32(1e30))
    else:
        assert np.all(s_o == floor_step)


# weight row lengths: 512 / 2048 / 4096 / 16384 (row kernel, one, two and four
# chunks per lane), 36864 (bf16 rows re-formed from the packed row), 65536
# (two-sweep kernel)
WEIGHT_K = [512, 2048, 4096, 16384, 36864, 65536]


@pytest.mark.parametrize("K", WEIGHT_K)
@pytest.mark.parametrize("w_mode", ["per_channel", "per_tensor"])
def test_weight_step_extremes(K, w_mode):
    """sq_calibrate at alpha = 1 with calibration peaks of exactly 1: s = 1
    (eq. (4): a^1 / w^0), so the smoothed weight rows are the rows themselves
    and their maxima span the finite range as the activation rows above."""
    d = dev()
    rng = np.random.default_rng(K + 5 + len(w_mode))
    xc = np.ones((3, K), np.float32)
    xc[1] = -1.0
    w = extreme_rows(rng, K, "bf16")
    xcb = to_bf16_bits(xc)
    say(f"[case] weight step extremes K={K} {w_mode}")
    cal = sq.sq_calibrate(to_dev(xcb, d), to_dev(w, d), 1.0, w_mode=w_mode)
    ref = oracle.calibrate(xcb, w, 1.0, w_per_tensor=(w_mode == "per_tensor"))
    assert np.all(ref["s"] == np.float32(1.0))
    assert_same("s", to_np(cal["s"]), ref["s"])
    assert_same("w_scale", to_np(cal["w_scale"]), ref["w_scale"])
    assert_same("wq", to_np(cal["wq"]), ref["wq"])
    if w_mode == "per_channel":
        ws = ref["w_scale"]
        assert ws[0] == np.float32(1e-7) / np.float32(127) and ws[1] == ws[0] and ws[6] == ws[0]
        assert ws[3] > np.float32(1e36) and ws[5] > np.float32(1e36)
