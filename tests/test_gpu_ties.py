"""Exact quantizer ties on the GPU, every element against the oracle.

[Review] §2.2 rounds x / Delta to the nearest integer without fixing the tie
rule; the library and the oracle round half to even (the [Edge] §三 listing's roundf rounds
half away from zero, and the two differ exactly at x / Delta = k + 1/2).
Random workload data almost never lands on a tie, so these inputs are built
to: steps that are powers of two (or 1.5 times one), smoothing factors that
are powers of two, and values (k + 1/2) * Delta for even and odd k, both signs,
up to the saturating +-127.5 and beyond.  Every kernel variant of each path
runs (row lengths pick the activation and weight kernels, shapes pick the GEMM
kernels), and every output element is compared bit for bit with the oracle:

  per-token, static and dynamic per-tensor activation codes (plain and
  LayerNorm mode), the smoothed per-output-channel and per-tensor weight codes
  (sq_calibrate at alpha = 1, where s is the calibration peak exactly), the
  int8 requantizing GEMM epilogue of sq_gemm_w8a8_ex, and bf16 outputs whose
  rounding is a tie.  Also the dequantization order on the GPU
  (tests/golden/dequant_order_example.txt).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values that are exactly representable."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    b = v.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def tie_values(rng, n, step, sat=False):
    """n smoothed values: 70% exact ties (k + 1/2) * step with k in [-127, 126]
    (even and odd k, both signs), the rest integer multiples k * step (|k| <=
    126); every value has at most 8 significant bits times step's.  sat: also
    +-127.5, +-128, +-200 and +-126.5 steps (static mode saturation)."""
    k = rng.integers(-127, 127, n)
    v = (k + 0.5) * step
    other = rng.integers(-126, 127, n) * step
    v = np.where(rng.random(n) < 0.7, v, other)
    if sat:
        extra = np.array([127.5, -127.5, 128.0, -128.0, 200.0, -200.0, 126.5, -126.5]) * step
        pos = rng.choice(n, size=min(n, len(extra)), replace=False)
        v[pos] = extra[: len(pos)]
    return v.astype(np.float32)


def count_ties(xhat, step):
    q = np.asarray(xhat, np.float64) / np.asarray(step, np.float64)
    return int(np.count_nonzero(np.abs(q - np.floor(q)) == 0.5))


def pow2_factors(rng, K):
    return (2.0 ** rng.integers(-2, 3, K)).astype(np.float32)


# row lengths that select every activation kernel: short rows packed in a wave
# (64, 128, 256), one row per block with cached factors (512, 4096, 16384),
# uncached rows (24576, 49152) and the multi-sweep kernel (65536)
PLAIN_K = [64, 128, 256, 512, 4096, 16384, 24576, 49152, 65536]


@pytest.mark.parametrize("K", PLAIN_K)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_per_token_ties(K, xdt):
    d = dev()
    rng = np.random.default_rng(K + (7 if xdt == "f32" else 0))
    M = 6
    # row peak 127 * 2^e, so the row's step is exactly 2^e
    e = rng.integers(-3, 4, M)
    step = (2.0 ** e).astype(np.float32)
    xh = np.stack([tie_values(rng, K, step[m]) for m in range(M)])
    for m in range(M):
        xh[m, rng.integers(K)] = 127.0 * step[m] * (1 if m % 2 else -1)
    s = pow2_factors(rng, K)
    x = (xh * s[None, :]).astype(np.float32)
    say(f"[case] per-token ties K={K} x={xdt}: {count_ties(xh, step[:, None])} ties")
    assert count_ties(xh, step[:, None]) > M * K // 3
    xin = bf16_bits(x) if xdt == "bf16" else x
    xq, xs = sq.sq_smooth_quantize_act(to_dev(xin, d), to_dev(s, d), mode="per_token")
    q_o, s_o, _ = oracle.smooth_quantize_act(xin, s=s)
    assert_same("x_scale", to_np(xs), s_o)
    assert np.array_equal(s_o, step)
    assert_same("xq", to_np(xq), q_o)


@pytest.mark.parametrize("K", PLAIN_K)
@pytest.mark.parametrize("step", [1.0, 0.25, 1.5])
def test_static_ties_and_saturation(K, step):
    """Static step 2^e or 1.5 * 2^e (fp32 input for 1.5: its ties need 10
    significant bits); quotients +-127.5 saturate to +-127, never -128."""
    d = dev()
    rng = np.random.default_rng(K + int(step * 8))
    M = 5
    xh = np.stack([tie_values(rng, K, step, sat=True) for _ in range(M)])
    s = pow2_factors(rng, K)
    x = (xh * s[None, :]).astype(np.float32)
    xin = bf16_bits(x) if step != 1.5 else x
    say(f"[case] static ties K={K} step={step}: {count_ties(xh, step)} ties")
    st = torch.tensor([step], dtype=torch.float32, device=d)
    xq, _ = sq.sq_smooth_quantize_act(to_dev(xin, d), to_dev(s, d), mode="static",
                                      static_scale=st)
    q_o, _, sat = oracle.smooth_quantize_act(xin, s=s, static=np.float32(step))
    assert sat > 0
    assert_same("xq", to_np(xq), q_o)
    assert to_np(xq).min() >= -127


@pytest.mark.parametrize("K", [128, 4096, 49152])
def test_dynamic_per_tensor_ties(K):
    d = dev()
    rng = np.random.default_rng(K + 3)
    M = 7
    xh = np.stack([tie_values(rng, K, 1.0) for _ in range(M)])
    xh[3, 5] = -127.0  # the batch peak: step exactly 1
    s = pow2_factors(rng, K)
    xin = bf16_bits(xh * s[None, :])
    say(f"[case] dynamic per-tensor ties K={K}: {count_ties(xh, 1.0)} ties")
    xq, xs = sq.sq_smooth_quantize_act(to_dev(xin, d), to_dev(s, d), mode="dynamic_per_tensor")
    q_o, s_o, _ = oracle.smooth_quantize_act(xin, s=s, dynamic_per_tensor=True)
    assert_same("x_scale", to_np(xs), s_o)
    assert np.float32(s_o).item() == 1.0
    assert_same("xq", to_np(xq), q_o)


# LayerNorm rows: one row in registers (512, 4096, 8192, 16384) and the
# multi-sweep kernel (24576)
@pytest.mark.parametrize("K", [512, 4096, 8192, 16384, 24576])
@pytest.mark.parametrize("mode", ["per_token", "static", "dynamic_per_tensor"])
def test_layernorm_ties(K, mode):
    """Folded LayerNorm ([Edge] §二): channels with gamma' = 0 emit
    RN(RN(d rho) * 0) + beta' = beta' exactly, so beta' = (k + 1/2) * step puts a
    tie on every such channel of every token; the other channels (gamma' =
    2^-7, |x^| < 2) are ordinary values.  One channel with beta' = 127 * step
    fixes the per-token (and batch) step."""
    d = dev()
    rng = np.random.default_rng(K + len(mode))
    M = 6
    step = 0.5
    tie_ch = rng.random(K) < 0.6
    g_s = np.where(tie_ch, 0.0, 2.0 ** -7).astype(np.float32)
    b_s = np.where(tie_ch, tie_values(rng, K, step, sat=(mode == "static")), 0.0).astype(np.float32)
    peak = int(np.flatnonzero(tie_ch)[0])
    b_s[peak] = 127.0 * step
    x = bf16_bits(np.clip(np.round(rng.normal(0, 1, (M, K)) * 16), -127, 127) / 16)
    say(f"[case] LayerNorm ties K={K} mode={mode}: {int(tie_ch.sum())} tie channels per token")
    st = torch.tensor([step], dtype=torch.float32, device=d) if mode == "static" else None
    xq, xs = sq.sq_smooth_quantize_act(to_dev(x, d), None, to_dev(g_s, d), to_dev(b_s, d), 1e-5,
                                       mode, st)
    q_o, s_o, _ = oracle.smooth_quantize_act(
        x, g_s=g_s, b_s=b_s, static=np.float32(step) if mode == "static" else None,
        dynamic_per_tensor=(mode == "dynamic_per_tensor"))
    if mode != "static":
        assert_same("x_scale", to_np(xs), s_o)
        assert np.all(np.asarray(s_o) == np.float32(step))
    assert_same("xq", to_np(xq), q_o)
    xh = oracle.act_ln(x, g_s, b_s)
    assert count_ties(xh, step) > M * int(tie_ch.sum()) // 2


# weight rows: 256, 1024, 8192, 40960 (one row per block) and 65536 (two sweeps)
@pytest.mark.parametrize("K", [256, 1024, 8192, 40960, 65536])
@pytest.mark.parametrize("w_mode", ["per_channel", "per_tensor"])
def test_weight_ties(K, w_mode):
    """sq_calibrate at alpha = 1: s_j equals the calibration peak a_j, chosen
    as powers of two, so W^ = RN(W s) is exact; W^ rows hold (k + 1/2) * 2^f
    and one +-127 * 2^f, so the step is exactly 2^f (per tensor: one f for
    every row) and half the codes are ties."""
    d = dev()
    rng = np.random.default_rng(K + len(w_mode))
    N = 40
    a = pow2_factors(rng, K)
    xc = np.stack([a, a * 0.5, -a * 0.75]).astype(np.float32)
    f = np.zeros(N, np.int64) if w_mode == "per_tensor" else rng.integers(-8, -2, N)
    wh = np.stack([tie_values(rng, K, 2.0 ** f[n]) for n in range(N)])
    for n in range(N):
        wh[n, rng.integers(K)] = (127.0 if n % 3 else -127.0) * 2.0 ** f[n]
    w = bf16_bits(wh / a[None, :])
    xcb = bf16_bits(xc)
    say(f"[case] weight ties K={K} {w_mode}: {count_ties(wh, 2.0 ** f[:, None])} ties")
    cal = sq.sq_calibrate(to_dev(xcb, d), to_dev(w, d), 1.0, w_mode=w_mode)
    ref = oracle.calibrate(xcb, w, 1.0, w_per_tensor=(w_mode == "per_tensor"))
    assert_same("s", to_np(cal["s"]), ref["s"])
    assert np.array_equal(ref["s"], a)
    assert_same("w_scale", to_np(cal["w_scale"]), ref["w_scale"])
    assert_same("wq", to_np(cal["wq"]), ref["wq"])
    assert_same("static_scale", to_np(cal["static_scale"])[0], ref["static_scale"])


# (M, N, K): ping-pong tiles (M > 64, K % 128 == 0), the short-K kernel
# (K <= 256), the decode kernel (M <= 64), the register-staged fallback
# (K % 128 != 0)
GEMM_SHAPES = [(300, 260, 512), (200, 300, 128), (40, 96, 1024), (130, 70, 192), (20, 33, 64)]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_requant_epilogue_ties(shape):
    """sq_gemm_w8a8_ex with int8 output ([Edge] §二: the next linear's smoothing
    and static quantization fused into this GEMM's epilogue).  dx = 1 and
    dw = 1/2 make y = acc / 2 exact; the bias is a multiple of 1/2 and s' * D
    is 1/2, 1 or 2, so y2 / (s' D) is a tie whenever the accumulator (plus
    twice the bias) has the right parity; rows scaled by 1, 2 or 3 push |y|
    past 127.5 D (saturation)."""
    d = dev()
    M, N, K = shape
    rng = np.random.default_rng(M * N + K)
    c = rng.integers(1, 4, M)[:, None]
    xq = (rng.integers(-2, 3, (M, K)) * c).astype(np.int8)
    wq = rng.integers(-2, 3, (N, K)).astype(np.int8)
    xs = np.ones(M, np.float32)
    ws = np.full(N, 0.5, np.float32)
    bias = (rng.integers(-20, 21, N) * 0.5).astype(np.float32)
    next_s = (2.0 ** rng.integers(0, 2, N)).astype(np.float32)
    say(f"[case] requant ties {M}x{N}x{K}")
    sat_total = 0
    for D, relu, use_s in [(1.0, False, False), (1.0, True, True), (0.5, True, True),
                           (0.5, False, True)]:
        y = sq.sq_gemm_w8a8_ex(to_dev(xq, d), to_dev(xs, d), to_dev(wq, d), to_dev(ws, d),
                               out_dtype="i8", bias=to_dev(bias, d), relu=relu,
                               next_s=to_dev(next_s, d) if use_s else None,
                               next_scale=torch.tensor([D], dtype=torch.float32, device=d))
        y2 = oracle.epilogue(oracle.dequant(oracle.gemm_i32(xq, wq), xs, ws), bias, relu)
        ns = next_s if use_s else np.ones(N, np.float32)
        ties = count_ties(y2 / ns[None, :], D)
        ref, sat = oracle.requant(y2, next_s if use_s else None, np.float32(D))
        sat_total += sat
        say(f"  D={D} relu={relu} s'={use_s}: {ties} ties, {sat} saturated")
        assert ties > 0
        assert_same(f"codes D={D} relu={relu} s'={use_s}", to_np(y), ref)
    assert sat_total > 0
    # bf16 outputs whose rounding is a tie: dw = 2^-8 makes y = acc / 256
    # exact, halfway between two bf16 values when its fp32 bits end in 0x8000
    xq_w = rng.integers(-127, 128, (M, K)).astype(np.int8)
    ws8 = np.full(N, 2.0 ** -8, np.float32)
    y = sq.sq_gemm_w8a8(to_dev(xq_w, d), to_dev(xs, d), to_dev(wq, d), to_dev(ws8, d),
                        out_dtype="bf16")
    y32 = oracle.dequant(oracle.gemm_i32(xq_w, wq), xs, ws8)
    n_ties = int(np.count_nonzero((y32.view(np.uint32) & 0xFFFF) == 0x8000))
    say(f"  bf16 rounding ties: {n_ties}")
    assert n_ties > 0
    assert_same("y[bf16]", to_np(y), oracle.f32_to_bf16(y32))


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_order_on_gpu(shape):
    """tests/golden/dequant_order_example.txt on every GEMM kernel: acc = 3,
    dx = dw = 1 + 2^-12 give fp32 bits 0x40401800 in the [Edge] §三 order
    (factor first), 0x40401801 in the other."""
    g = {}
    for line in open(os.path.join(GOLDEN, "dequant_order_example.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=", 1)
            g[k.strip()] = v.strip()
    d = dev()
    M, N, K = shape
    xq = np.zeros((M, K), np.int8)
    wq = np.zeros((N, K), np.int8)
    xq[:, :3] = 1
    wq[:, :3] = 1
    dx = np.array([int(g["dx_bits"], 16)], np.uint32).view(np.float32)
    dw = np.array([int(g["dw_bits"], 16)], np.uint32).view(np.float32)
    say(f"[case] dequant order {M}x{N}x{K}")
    for mode, w_mode, xs, ws in [("per_token", "per_channel", np.repeat(dx, M), np.repeat(dw, N)),
                                 ("static", "per_tensor", dx, dw)]:
        y = sq.sq_gemm_w8a8(to_dev(xq, d), to_dev(xs, d), to_dev(wq, d), to_dev(ws, d), mode,
                            "f32", w_mode=w_mode)
        bits = to_np(y).view(np.uint32)
        assert np.all(bits == int(g["y_bits"], 16)), (mode, hex(int(bits.ravel()[0])))
