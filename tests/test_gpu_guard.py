"""Guard bands: no kernel writes outside its outputs.

Every output of every call is placed inside a larger device buffer whose
margins (4 KiB before and after) hold a sentinel byte; after the call the
margins must be untouched, and the output itself must equal that of the same
call into freshly allocated tensors (the parity tests compare those with the
oracle).  Shapes are ragged in M and N (rows of odd byte length, partial
tiles) and pick every GEMM kernel -- ping-pong 256x128, 256x256 and the mixed
launch, short K, the decode kernel and both register-staged fallbacks, plus the
batched product -- every activation-quantizer kernel (short rows packed in a
wave, cached and uncached rows, the long-row kernel with lanes past the
row's end, the multi-sweep kernel, LayerNorm variants; per-token, static and
dynamic per-tensor), the calibration kernels (weight
rows of every length, per channel and per tensor, with and without the
LayerNorm fold) and the robust-calibration calls.
"""
import ctypes

import numpy as np
import pytest
import torch

import w8a8_int8_gemm_colwise_amd as sq
from sqcase import dev, say

pytestmark = pytest.mark.gpu

PAD = 4096
SENT = 0xA5


class Guarded:
    """A tensor of `shape` / `dtype` at offset PAD of a sentinel-filled buffer."""

    def __init__(self, shape, dtype, d):
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * torch.tensor([], dtype=dtype).element_size()
        self.buf = torch.full((2 * PAD + self.nbytes,), SENT, dtype=torch.uint8, device=d)
        self.t = self.buf[PAD:PAD + self.nbytes].view(dtype).view(shape)

    def check(self, name):
        head = self.buf[:PAD]
        tail = self.buf[PAD + self.nbytes:]
        bad_h = int((head != SENT).sum())
        bad_t = int((tail != SENT).sum())
        assert bad_h == 0 and bad_t == 0, f"{name}: {bad_h} bytes before, {bad_t} after changed"


def same(name, a, b):
    """Equal shapes, dtypes and bytes (a bitwise comparison: -0 differs from +0)."""
    assert a.shape == b.shape and a.dtype == b.dtype, name
    assert torch.equal(a.reshape(-1).view(torch.uint8), b.reshape(-1).view(torch.uint8)), name


def rand_codes(rng, rows, K, d):
    return torch.from_numpy(rng.integers(-127, 128, (rows, K)).astype(np.int8)).to(d)


# (M, N, K, kernel)
GEMMS = [
    (300, 259, 512, "ping-pong 256x128"),
    (2000, 8100, 384, "ping-pong 256x256"),
    (2000, 12000, 384, "mixed 256x256 + 256x128"),
    (200, 301, 64, "short K 64"),
    (129, 257, 128, "short K 128"),
    (300, 131, 256, "short K 256"),
    (40, 1001, 1024, "decode, two 32-row tiles"),
    (20, 70, 256, "decode, one 32-row tile"),
    (33, 70, 192, "register-staged, M <= 64"),
    (130, 70, 192, "register-staged 128x128"),
    (2000, 8100, 320, "register-staged 256x128"),
]


@pytest.mark.parametrize("case", GEMMS, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
def test_gemm_outputs_stay_in_bounds(case):
    M, N, K, kern = case
    d = dev()
    rng = np.random.default_rng(M + N + K)
    xq, wq = rand_codes(rng, M, K, d), rand_codes(rng, N, K, d)
    xs = torch.from_numpy(rng.uniform(1e-3, 1e-2, M).astype(np.float32)).to(d)
    ws = torch.from_numpy(rng.uniform(1e-4, 1e-3, N).astype(np.float32)).to(d)
    bias = torch.from_numpy(rng.normal(0, 1, N).astype(np.float32)).to(d)
    ns = torch.from_numpy(rng.uniform(0.5, 2, N).astype(np.float32)).to(d)
    step = torch.tensor([0.02], dtype=torch.float32, device=d)
    say(f"[case] guard GEMM {M}x{N}x{K} ({kern})")
    for out, dt in [("f32", torch.float32), ("bf16", torch.bfloat16), ("i32", torch.int32)]:
        g = Guarded((M, N), dt, d)
        ref = sq.sq_gemm_w8a8(xq, xs, wq, ws, out_dtype=out)
        sq.sq_gemm_w8a8(xq, xs, wq, ws, out_dtype=out, y=g.t)
        torch.cuda.synchronize()
        g.check(f"y[{out}]")
        same(f"y[{out}]", g.t, ref)
    # fused epilogues: bias + ReLU (bf16), and int8 codes for the next linear
    g = Guarded((M, N), torch.bfloat16, d)
    ref = sq.sq_gemm_w8a8_ex(xq, xs, wq, ws, out_dtype="bf16", bias=bias, relu=True)
    sq.sq_gemm_w8a8_ex(xq, xs, wq, ws, out_dtype="bf16", bias=bias, relu=True, y=g.t)
    g8 = Guarded((M, N), torch.int8, d)
    ref8 = sq.sq_gemm_w8a8_ex(xq, xs, wq, ws, out_dtype="i8", next_s=ns, next_scale=step)
    sq.sq_gemm_w8a8_ex(xq, xs, wq, ws, out_dtype="i8", next_s=ns, next_scale=step, y=g8.t)
    torch.cuda.synchronize()
    g.check("y[bf16, bias, relu]")
    g8.check("y[i8]")
    same("y[bf16, bias, relu]", g.t, ref)
    same("y[i8]", g8.t, ref8)


@pytest.mark.parametrize("K", [128, 512])
def test_batched_outputs_stay_in_bounds(K):
    """Entries of 100 x 77 outputs: no entry after the first starts on a
    16-byte boundary (element-wise stores)."""
    d = dev()
    B, M, N = 3, 100, 77
    rng = np.random.default_rng(K)
    xq = torch.from_numpy(rng.integers(-127, 128, (B, M, K)).astype(np.int8)).to(d)
    wq = torch.from_numpy(rng.integers(-127, 128, (B, N, K)).astype(np.int8)).to(d)
    xs = torch.from_numpy(rng.uniform(1e-3, 1e-2, (B, M)).astype(np.float32)).to(d)
    ws = torch.from_numpy(rng.uniform(1e-3, 1e-2, (B, N)).astype(np.float32)).to(d)
    say(f"[case] guard batched {B}x{M}x{N}x{K}")
    for out, dt in [("f32", torch.float32), ("bf16", torch.bfloat16), ("i32", torch.int32)]:
        g = Guarded((B, M, N), dt, d)
        ref = sq.sq_bmm_w8a8(xq, xs, wq, ws, out_dtype=out)
        sq.sq_bmm_w8a8(xq, xs, wq, ws, out_dtype=out, y=g.t)
        torch.cuda.synchronize()
        g.check(f"y[{out}]")
        same(f"y[{out}]", g.t, ref)


ACT_K = [64, 128, 256, 512, 4096, 16384, 16448, 24576, 32832, 49152, 65536]


@pytest.mark.parametrize("K", ACT_K)
@pytest.mark.parametrize("mode", ["per_token", "static", "dynamic_per_tensor"])
def test_activation_quantizer_stays_in_bounds(K, mode):
    d = dev()
    M = 37
    rng = np.random.default_rng(K + len(mode))
    x = torch.from_numpy(rng.normal(0, 1, (M, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    s = torch.from_numpy(rng.uniform(0.5, 2, K).astype(np.float32)).to(d)
    st = torch.tensor([0.01], dtype=torch.float32, device=d)
    say(f"[case] guard act quant M={M} K={K} {mode}")
    ref_q, ref_s = sq.sq_smooth_quantize_act(x, s, mode=mode, static_scale=st)
    gq = Guarded((M, K), torch.int8, d)
    ns = {"per_token": M, "dynamic_per_tensor": 1}.get(mode)
    gs = Guarded((ns,), torch.float32, d) if ns else None
    sq.sq_smooth_quantize_act(x, s, mode=mode, static_scale=st, xq=gq.t,
                              x_scale=gs.t if gs else None)
    torch.cuda.synchronize()
    gq.check("xq")
    same("xq", gq.t, ref_q)
    if gs:
        gs.check("x_scale")
        same("x_scale", gs.t, ref_s)


@pytest.mark.parametrize("K", [512, 4096, 8192, 10240, 14400, 16384, 24576])
@pytest.mark.parametrize("mode", ["per_token", "static", "dynamic_per_tensor"])
def test_layernorm_quantizer_stays_in_bounds(K, mode):
    d = dev()
    M = 13
    rng = np.random.default_rng(K + 2 * len(mode))
    x = torch.from_numpy(rng.normal(0, 1, (M, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    g = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32)).to(d)
    b = torch.from_numpy(rng.normal(0, 0.1, K).astype(np.float32)).to(d)
    st = torch.tensor([0.02], dtype=torch.float32, device=d)
    say(f"[case] guard LayerNorm quant M={M} K={K} {mode}")
    ref_q, ref_s = sq.sq_smooth_quantize_act(x, None, g, b, 1e-5, mode, st)
    gq = Guarded((M, K), torch.int8, d)
    ns = {"per_token": M, "dynamic_per_tensor": 1}.get(mode)
    gs = Guarded((ns,), torch.float32, d) if ns else None
    sq.sq_smooth_quantize_act(x, None, g, b, 1e-5, mode, st, xq=gq.t, x_scale=gs.t if gs else None)
    torch.cuda.synchronize()
    gq.check("xq")
    same("xq", gq.t, ref_q)
    if gs:
        gs.check("x_scale")
        same("x_scale", gs.t, ref_s)


# weight rows of 256 .. 65536 elements (every weight-quantizer kernel); N odd
@pytest.mark.parametrize("K", [256, 1024, 8192, 40960, 65536])
@pytest.mark.parametrize("variant", ["per_channel", "per_tensor", "layernorm"])
def test_calibration_stays_in_bounds(K, variant):
    d = dev()
    N, T = 37, 5
    rng = np.random.default_rng(K + len(variant))
    xc = torch.from_numpy(rng.normal(0, 1, (T, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    w = torch.from_numpy(rng.normal(0, 0.02, (N, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    ln = variant == "layernorm"
    gam = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32)).to(d) if ln else None
    bet = torch.from_numpy(rng.normal(0, 0.1, K).astype(np.float32)).to(d) if ln else None
    w_mode = "per_tensor" if variant == "per_tensor" else "per_channel"
    say(f"[case] guard calibrate N={N} K={K} {variant}")
    ref = sq.sq_calibrate(xc, w, 0.5, gam, bet, w_mode=w_mode)
    shapes = {"s": (K,), "wq": (N, K), "w_scale": (N if w_mode == "per_channel" else 1,),
              "static_scale": (1,), "x_absmax": (K,), "w_absmax": (K,)}
    if ln:
        shapes.update(ln_gamma_s=(K,), ln_beta_s=(K,))
    gd = {k: Guarded(v, torch.int8 if k == "wq" else torch.float32, d) for k, v in shapes.items()}
    sq.sq_calibrate(xc, w, 0.5, gam, bet, out={k: v.t for k, v in gd.items()}, w_mode=w_mode)
    torch.cuda.synchronize()
    for k, gg in gd.items():
        gg.check(k)
        same(k, gg.t, ref[k])


def test_robust_calls_stay_in_bounds():
    """Channel quantile (output and a workspace of exactly the queried size),
    clip counts, and the alpha search's outputs and workspace."""
    d = dev()
    L = sq.lib()
    rng = np.random.default_rng(77)
    T, K, N = 300, 1024, 129
    x = torch.from_numpy(rng.normal(0, 1, (T, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    w = torch.from_numpy(rng.normal(0, 0.02, (N, K)).astype(np.float32)).to(d).to(torch.bfloat16)
    stream = torch.cuda.current_stream(d).cuda_stream
    say("[case] guard channel quantile / clip count / alpha search")
    ref = sq.sq_channel_quantile(x, 0.9)
    nb = L.sq_channel_quantile_workspace_size(K)
    go, gw = Guarded((K,), torch.float32, d), Guarded((nb,), torch.uint8, d)
    sq.sq_channel_quantile(x, 0.9, out=go.t, workspace=gw.t)
    torch.cuda.synchronize()
    go.check("quantile out")
    gw.check("quantile workspace")
    same("quantile", go.t, ref)

    s = torch.from_numpy(rng.uniform(0.5, 2, K).astype(np.float32)).to(d)
    st = torch.tensor([0.005], dtype=torch.float32, device=d)
    ref_c, ref_pc = sq.sq_clip_count(x, st, s=s, per_channel=True)
    gc, gpc = Guarded((1,), torch.int64, d), Guarded((K,), torch.int32, d)
    rc = L.sq_clip_count(x.data_ptr(), sq.SQ_BF16, T, K, s.data_ptr(), None, None, 1e-5,
                         st.data_ptr(), gc.t.data_ptr(), gpc.t.data_ptr(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    gc.check("clip count")
    gpc.check("clip per channel")
    same("clip count", gc.t, ref_c)
    same("clip per channel", gpc.t, ref_pc)

    alphas = [0.25, 0.5, 0.75]
    ref_e, ref_we, ref_b = sq.sq_alpha_search(x, w, alphas)
    nb = L.sq_alpha_search_workspace_size(T, N, K)
    ge, gwe = Guarded((3,), torch.float64, d), Guarded((3,), torch.float64, d)
    gb, gws = Guarded((1,), torch.int32, d), Guarded((nb,), torch.uint8, d)
    al = (ctypes.c_float * 3)(*alphas)
    rc = L.sq_alpha_search(x.data_ptr(), sq.SQ_BF16, T, w.data_ptr(), sq.SQ_BF16, N, K,
                           ctypes.addressof(al), 3, sq.SQ_PER_TOKEN, sq.SQ_W_PER_CHANNEL,
                           ge.t.data_ptr(), gwe.t.data_ptr(), gb.t.data_ptr(), gws.t.data_ptr(),
                           nb, stream)
    assert rc == 0
    torch.cuda.synchronize()
    for name, gg, r in [("err", ge, ref_e), ("werr", gwe, ref_we), ("best", gb, ref_b)]:
        gg.check(name)
        same(name, gg.t, r)
    gws.check("alpha workspace")
