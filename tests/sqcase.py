"""Shared plumbing for the GPU parity tests: move seeded inputs to the GPU, run
the library's three calls through the C ABI binding, and run the oracle on the
same inputs (in full, or on sampled rows/columns at full sizes)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, d) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(d)
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def sample_idx(n: int, k: int, seed: int) -> np.ndarray:
    """k sorted indices of range(n) that always include 0 and n-1."""
    if n <= k:
        return np.arange(n, dtype=np.int64)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid])).astype(np.int64)


_C5 = {}


def c5_inputs():
    """The LayerNorm pipeline workload (hidden 8192, 65536 calibration tokens),
    generated once per process."""
    if not _C5:
        spec = datagen.workload(5).layers[0]
        _C5["xc"] = datagen.calibration_x(spec)
        _C5["w"] = datagen.weights(spec)
        _C5["x"] = datagen.eval_x(spec)
        _C5["gb"] = datagen.ln_params(spec)
    return _C5


def gpu_calibrate(x_cal, w, alpha, gamma=None, beta=None, w_mode="per_channel"):
    d = dev()
    xt, wt = to_dev(x_cal, d), to_dev(w, d)
    gt = None if gamma is None else to_dev(gamma, d)
    bt = None if beta is None else to_dev(beta, d)
    out = sq.sq_calibrate(xt, wt, alpha, gt, bt, w_mode=w_mode)
    del xt
    return out, wt


def assert_same(name, gpu, ref):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    if gpu.dtype.kind == "f":
        eq = (gpu.view(np.uint32 if gpu.dtype == np.float32 else gpu.dtype) ==
              ref.astype(gpu.dtype).view(np.uint32 if gpu.dtype == np.float32 else gpu.dtype))
    else:
        eq = gpu == ref
    bad = np.size(eq) - int(np.count_nonzero(eq))
    if bad:
        idx = np.argwhere(~eq)[:5]
        detail = [(tuple(int(v) for v in i), gpu[tuple(i)], ref[tuple(i)]) for i in idx]
        raise AssertionError(f"{name}: {bad} of {eq.size} differ; first {detail}")


def run_layer(spec: datagen.LayerSpec, x_cal, w, x, mode: str, n_rows: int | None = None,
              n_cols: int | None = None, seed: int = 0, out_kinds=("bf16", "f32", "i32"),
              gamma=None, beta=None, alpha=None, w_mode="per_channel"):
    """Run the whole path on the GPU and compare with the oracle.

    mode: activation step "per_token" | "static" | "dynamic_per_tensor";
    w_mode: weight step "per_channel" | "per_tensor".
    n_rows / n_cols: sample sizes of tokens / output channels for the
    element-wise comparison of per-row outputs (None = all).  The per-tensor
    steps need every row, so the oracle then quantizes in full and the
    comparison samples."""
    alpha = spec.alpha if alpha is None else alpha
    M, K = x.shape
    N = w.shape[0]
    wpt = w_mode == "per_tensor"
    say(f"[case] {spec.name} M={M} N={N} K={K} alpha={alpha} mode={mode} w_mode={w_mode} "
        f"ln={spec.ln}")
    # ---- GPU
    cal, wt = gpu_calibrate(x_cal, w, alpha, gamma, beta, w_mode=w_mode)
    d = dev()
    xt = to_dev(x, d)
    if spec.ln:
        xq_t, xs_t = sq.sq_smooth_quantize_act(xt, None, cal["ln_gamma_s"], cal["ln_beta_s"],
                                               1e-5, mode, cal["static_scale"])
    else:
        xq_t, xs_t = sq.sq_smooth_quantize_act(xt, cal["s"], mode=mode,
                                               static_scale=cal["static_scale"])
    ys = {k: sq.sq_gemm_w8a8(xq_t, xs_t, cal["wq"], cal["w_scale"], mode, k, w_mode=w_mode)
          for k in out_kinds}
    torch.cuda.synchronize()
    say("  gpu done")

    # ---- oracle on the same inputs
    a = oracle.colmax(x_cal)
    wm = oracle.colmax(w)
    s = oracle.smooth_factor(a, wm, alpha)
    assert_same("x_absmax", to_np(cal["x_absmax"]), a)
    assert_same("w_absmax", to_np(cal["w_absmax"]), wm)
    assert_same("s", to_np(cal["s"]), s)
    st = oracle.static_scale(a, s)
    assert_same("static_scale", to_np(cal["static_scale"])[0], st)
    gs = bs = None
    if spec.ln:
        gs, bs = oracle.ln_fold(gamma, beta, s)
        assert_same("ln_gamma_s", to_np(cal["ln_gamma_s"]), gs)
        assert_same("ln_beta_s", to_np(cal["ln_beta_s"]), bs)

    cols = None if n_cols is None else sample_idx(N, n_cols, seed + 1)
    rows = None if n_rows is None else sample_idx(M, n_rows, seed + 2)
    wq_g = to_np(cal["wq"])
    wsc_g = to_np(cal["w_scale"])
    if wpt:
        wq_o, wsc_o = oracle.weight_quant_per_tensor(w, s)
        if cols is not None:
            wq_o = wq_o[cols]
    else:
        wq_o, wsc_o = oracle.weight_quant(w, s, rows=cols)
        if cols is not None:
            wsc_g = wsc_g[cols]
    if cols is not None:
        wq_g = wq_g[cols]
    assert_same("w_scale", wsc_g, wsc_o)
    assert_same("wq", wq_g, wq_o)

    static = st if mode == "static" else None
    dyn_t = mode == "dynamic_per_tensor"
    act_rows = None if dyn_t else rows
    if spec.ln:
        xq_o, xs_o, sat = oracle.smooth_quantize_act(x, g_s=gs, b_s=bs, static=static,
                                                     rows=act_rows, dynamic_per_tensor=dyn_t)
    else:
        xq_o, xs_o, sat = oracle.smooth_quantize_act(x, s=s, static=static, rows=act_rows,
                                                     dynamic_per_tensor=dyn_t)
    if dyn_t and rows is not None:
        xq_o = xq_o[rows]
    xq_g = to_np(xq_t)
    xs_g = to_np(xs_t)
    if rows is not None:
        xq_g = xq_g[rows]
        if mode == "per_token":
            xs_g = xs_g[rows]
    assert_same("xq", xq_g, xq_o)
    assert_same("x_scale", xs_g, xs_o)

    acc = oracle.gemm_i32(xq_o, wq_o)
    per_token = mode == "per_token"
    y32 = oracle.dequant(acc, xs_o, wsc_o, per_token=per_token, w_per_tensor=wpt)
    refs = {"i32": acc, "f32": y32, "bf16": oracle.f32_to_bf16(y32)}
    for k, yt in ys.items():
        yg = to_np(yt)
        if rows is not None:
            yg = yg[rows]
        if cols is not None:
            yg = yg[:, cols]
        assert_same(f"y[{k}]", yg, refs[k])
    say(f"  parity ok (saturated codes: {sat})")
    return dict(cal=cal, xq=xq_t, xs=xs_t, ys=ys, s=s, sat=sat)
