"""Python binding of libsq.so, the MI355X (gfx950) SmoothQuant W8A8 library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory (output tensors are allocated with
``torch.empty`` on the input's device) and the current HIP stream.  The
functions carry the C ABI's names (include/sq.h):

  sq_calibrate            offline: column absmax of X_cal and W, eq. (4)
                          smoothing factor, LayerNorm fold, static scale,
                          smoothed per-output-channel int8 weights
  sq_smooth_quantize_act  runtime: X/s (or the folded LayerNorm), then
                          per-token or static per-tensor int8
  sq_gemm_w8a8            runtime: int8 GEMM, int32 accumulation, dequant
  sq_gemm_w8a8_ex         the same with the fused epilogue (bias, ReLU, int8
                          codes for the next linear)
  sq_bmm_w8a8             batched int8 GEMM (the attention products)
  sq_channel_quantile     robust per-channel activation statistic
  sq_channel_quantile_noalloc  the same without a workspace (no allocation)
  sq_calibrate_stat       the offline half from a given activation statistic
  sq_clip_count           saturation count of the static quantizer
  sq_alpha_search         candidate alphas: output and weight errors

There is no fallback: if libsq.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsq.so")

SQ_F32, SQ_BF16, SQ_I8, SQ_I32 = 0, 1, 2, 3
SQ_PER_TOKEN, SQ_STATIC_PER_TENSOR, SQ_DYNAMIC_PER_TENSOR = 0, 1, 2
SQ_W_PER_CHANNEL, SQ_W_PER_TENSOR = 0, 1
SQ_MAX_K = 133120
SQ_ABI_VERSION = 4
SQ_NOALLOC_MAX_K = 16384

# The SmoothQuant efficiency levels ([Review] §6.3): (weight mode, activation
# mode).  "colwise" is the per-output-channel weight path with per-token
# activations.
SETTINGS = {
    "colwise": ("per_channel", "per_token"),
    "O1": ("per_tensor", "per_token"),
    "O2": ("per_tensor", "dynamic_per_tensor"),
    "O3": ("per_tensor", "static"),
}
EXPORTED = ("sq_calibrate", "sq_smooth_quantize_act", "sq_gemm_w8a8", "sq_gemm_w8a8_ex",
            "sq_bmm_w8a8", "sq_channel_quantile_workspace_size", "sq_channel_quantile",
            "sq_channel_quantile_noalloc", "sq_calibrate_stat", "sq_clip_count",
            "sq_alpha_search_workspace_size",
            "sq_alpha_search", "sq_status_string", "sq_abi_version")


class SqEpilogue(ctypes.Structure):
    """struct sq_epilogue of sq.h (fused epilogue of sq_gemm_w8a8_ex)."""
    _fields_ = [("bias", ctypes.c_void_p), ("next_s", ctypes.c_void_p),
                ("next_scale", ctypes.c_void_p), ("relu", ctypes.c_int)]

_lib = None


class SQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsq.so (built by ``python -m w8a8_int8_gemm_colwise_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m w8a8_int8_gemm_colwise_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.sq_calibrate.restype = ci
    L.sq_calibrate.argtypes = [vp, ci, i64, vp, ci, i64, i64, cf, ci, vp, vp, vp, vp, vp, vp, vp,
                               vp, vp, vp, vp]
    L.sq_smooth_quantize_act.restype = ci
    L.sq_smooth_quantize_act.argtypes = [vp, ci, i64, i64, vp, vp, vp, cf, ci, vp, vp, vp, vp]
    L.sq_gemm_w8a8.restype = ci
    L.sq_gemm_w8a8.argtypes = [vp, vp, ci, vp, vp, ci, i64, i64, i64, vp, ci, vp]
    L.sq_gemm_w8a8_ex.restype = ci
    L.sq_gemm_w8a8_ex.argtypes = [vp, vp, ci, vp, vp, ci, i64, i64, i64,
                                  ctypes.POINTER(SqEpilogue), vp, ci, vp]
    L.sq_bmm_w8a8.restype = ci
    L.sq_bmm_w8a8.argtypes = [vp, i64, vp, i64, ci, vp, i64, vp, i64, ci, i64, i64, i64, i64,
                              vp, i64, ci, vp]
    sz = ctypes.c_size_t
    L.sq_channel_quantile_workspace_size.restype = sz
    L.sq_channel_quantile_workspace_size.argtypes = [i64]
    L.sq_channel_quantile.restype = ci
    L.sq_channel_quantile.argtypes = [vp, ci, i64, i64, cf, vp, vp, sz, vp]
    L.sq_channel_quantile_noalloc.restype = ci
    L.sq_channel_quantile_noalloc.argtypes = [vp, ci, i64, i64, cf, vp, vp]
    L.sq_calibrate_stat.restype = ci
    L.sq_calibrate_stat.argtypes = [vp, vp, ci, i64, i64, cf, ci, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp]
    L.sq_clip_count.restype = ci
    L.sq_clip_count.argtypes = [vp, ci, i64, i64, vp, vp, vp, cf, vp, vp, vp, vp]
    L.sq_alpha_search_workspace_size.restype = sz
    L.sq_alpha_search_workspace_size.argtypes = [i64, i64, i64]
    L.sq_alpha_search.restype = ci
    L.sq_alpha_search.argtypes = [vp, ci, i64, vp, ci, i64, i64, vp, ci, ci, ci, vp, vp, vp, vp,
                                  sz, vp]
    L.sq_status_string.restype = ctypes.c_char_p
    L.sq_status_string.argtypes = [ci]
    L.sq_abi_version.restype = ci
    L.sq_abi_version.argtypes = []
    if L.sq_abi_version() != SQ_ABI_VERSION:
        raise RuntimeError("libsq.so ABI version mismatch")
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise SQError(rc, lib().sq_status_string(rc).decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    raise TypeError(f"activation/weight dtype must be float32 or bfloat16, got {t.dtype}")


def _dev2d(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")


def _vec(t: torch.Tensor | None, n, name: str, device, dtype=torch.float32):
    """A caller-supplied vector (input or output): contiguous, on ``device``, of
    ``dtype`` and with exactly ``n`` elements (or one of the counts in ``n``)."""
    if t is None:
        return
    counts = n if isinstance(n, tuple) else (n,)
    if (not t.is_cuda or t.device != device or t.dtype != dtype or not t.is_contiguous()
            or t.numel() not in counts):
        want = " or ".join(str(c) for c in counts)
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of {want} elements "
                         f"on {device}")


def _out2d(t: torch.Tensor, rows: int, cols: int, name: str, device, dtype):
    """A caller-supplied 2-D output: contiguous [rows, cols] of ``dtype`` on ``device``."""
    if (not t.is_cuda or t.device != device or t.dtype != dtype or not t.is_contiguous()
            or tuple(t.shape) != (rows, cols)):
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape "
                         f"[{rows}, {cols}] on {device}")


def _mode(mode) -> int:
    if mode in ("per_token", SQ_PER_TOKEN):
        return SQ_PER_TOKEN
    if mode in ("static", SQ_STATIC_PER_TENSOR):
        return SQ_STATIC_PER_TENSOR
    if mode in ("dynamic_per_tensor", SQ_DYNAMIC_PER_TENSOR):
        return SQ_DYNAMIC_PER_TENSOR
    raise ValueError(f"unknown activation mode {mode!r}")


def _wmode(mode) -> int:
    if mode in ("per_channel", SQ_W_PER_CHANNEL):
        return SQ_W_PER_CHANNEL
    if mode in ("per_tensor", SQ_W_PER_TENSOR):
        return SQ_W_PER_TENSOR
    raise ValueError(f"unknown weight mode {mode!r}")


def sq_calibrate(x_cal: torch.Tensor, w: torch.Tensor, alpha: float,
                 ln_gamma: torch.Tensor | None = None, ln_beta: torch.Tensor | None = None,
                 out: dict | None = None, w_mode="per_channel") -> dict:
    """Offline half: returns dict(s, wq, w_scale, static_scale, x_absmax, w_absmax
    [, ln_gamma_s, ln_beta_s]).  ``out`` may supply preallocated tensors.
    w_mode "per_channel" (w_scale [N]) or "per_tensor" (w_scale [1])."""
    wm = _wmode(w_mode)
    _dev2d(x_cal, "x_cal")
    _dev2d(w, "w")
    T, K = x_cal.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("x_cal and w disagree on K")
    dev = w.device
    if x_cal.device != dev:
        raise ValueError("x_cal and w must be on one device")
    _vec(ln_gamma, K, "ln_gamma", dev)
    _vec(ln_beta, K, "ln_beta", dev)
    o = dict(out or {})
    f32 = dict(dtype=torch.float32, device=dev)
    nws = N if wm == SQ_W_PER_CHANNEL else 1
    vecs = {"s": K, "w_scale": nws, "static_scale": 1, "x_absmax": K, "w_absmax": K}
    if ln_gamma is not None:
        vecs.update(ln_gamma_s=K, ln_beta_s=K)
    for k, n in vecs.items():
        if k in o:
            _vec(o[k], n, f"out[{k!r}]", dev)
        else:
            o[k] = torch.empty(n, **f32)
    if "wq" in o:
        _out2d(o["wq"], N, K, "out['wq']", dev, torch.int8)
    else:
        o["wq"] = torch.empty((N, K), dtype=torch.int8, device=dev)
    _check(lib().sq_calibrate(
        _ptr(x_cal), _dt(x_cal), T, _ptr(w), _dt(w), N, K, float(alpha), wm,
        _ptr(ln_gamma), _ptr(ln_beta), _ptr(o["s"]), _ptr(o["wq"]), _ptr(o["w_scale"]),
        _ptr(o["static_scale"]), _ptr(o.get("ln_gamma_s")), _ptr(o.get("ln_beta_s")),
        _ptr(o["x_absmax"]), _ptr(o["w_absmax"]), _stream(dev)))
    return o


def sq_smooth_quantize_act(x: torch.Tensor, s: torch.Tensor | None = None,
                           ln_gamma_s: torch.Tensor | None = None,
                           ln_beta_s: torch.Tensor | None = None, ln_eps: float = 1e-5,
                           mode="per_token", static_scale: torch.Tensor | None = None,
                           xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None):
    """Runtime activation side: returns (xq int8 [M,K], the step(s)): x_scale
    fp32 [M] per token, the batch step [1] for "dynamic_per_tensor", or the
    static scale [1]."""
    _dev2d(x, "x")
    M, K = x.shape
    md = _mode(mode)
    dev = x.device
    _vec(s, K, "s", dev)
    _vec(ln_gamma_s, K, "ln_gamma_s", dev)
    _vec(ln_beta_s, K, "ln_beta_s", dev)
    if md == SQ_STATIC_PER_TENSOR:
        _vec(static_scale, 1, "static_scale", dev)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    else:
        _out2d(xq, M, K, "xq", dev, torch.int8)
    if md != SQ_STATIC_PER_TENSOR:
        n = M if md == SQ_PER_TOKEN else 1
        if x_scale is None:
            x_scale = torch.empty(n, dtype=torch.float32, device=dev)
        else:
            _vec(x_scale, n, "x_scale", dev)
    _check(lib().sq_smooth_quantize_act(
        _ptr(x), _dt(x), M, K, _ptr(s), _ptr(ln_gamma_s), _ptr(ln_beta_s), float(ln_eps), md,
        _ptr(static_scale) if md == SQ_STATIC_PER_TENSOR else None, _ptr(xq),
        _ptr(x_scale) if md != SQ_STATIC_PER_TENSOR else None, _stream(x.device)))
    return xq, (static_scale if md == SQ_STATIC_PER_TENSOR else x_scale)


_OUT = {"f32": (SQ_F32, torch.float32), "bf16": (SQ_BF16, torch.bfloat16),
        "i32": (SQ_I32, torch.int32), "i8": (SQ_I8, torch.int8)}


def _gemm_args(xq, x_scale, wq, w_scale, md, wm, code, tdt, y):
    """Shapes of a GEMM call; checks the scales and a caller-supplied output."""
    _dev2d(xq, "xq")
    _dev2d(wq, "wq")
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("xq and wq disagree on K")
    dev = xq.device
    if wq.device != dev:
        raise ValueError("xq and wq must be on one device")
    if code != SQ_I32:
        _vec(x_scale, M if md == SQ_PER_TOKEN else 1, "x_scale", dev)
        _vec(w_scale, N if wm == SQ_W_PER_CHANNEL else 1, "w_scale", dev)
    if y is None:
        y = torch.empty((M, N), dtype=tdt, device=dev)
    else:
        _out2d(y, M, N, "y", dev, tdt)
    return M, N, K, y


def sq_gemm_w8a8(xq: torch.Tensor, x_scale: torch.Tensor | None, wq: torch.Tensor,
                 w_scale: torch.Tensor | None, mode="per_token", out_dtype: str = "bf16",
                 y: torch.Tensor | None = None, w_mode="per_channel") -> torch.Tensor:
    """Int8 GEMM + dequant: y[M,N] = RN(float(acc) * RN(dx_t * dw_n)); mode is
    the activation step granularity, w_mode the weight's."""
    code, tdt = _OUT[out_dtype]
    md, wm = _mode(mode), _wmode(w_mode)
    M, N, K, y = _gemm_args(xq, x_scale, wq, w_scale, md, wm, code, tdt, y)
    _check(lib().sq_gemm_w8a8(_ptr(xq), _ptr(x_scale), md, _ptr(wq), _ptr(w_scale),
                              wm, M, N, K, _ptr(y), code, _stream(xq.device)))
    return y


def sq_gemm_w8a8_ex(xq: torch.Tensor, x_scale: torch.Tensor | None, wq: torch.Tensor,
                    w_scale: torch.Tensor | None, mode="per_token", out_dtype: str = "bf16",
                    y: torch.Tensor | None = None, w_mode="per_channel",
                    bias: torch.Tensor | None = None, relu: bool = False,
                    next_s: torch.Tensor | None = None,
                    next_scale: torch.Tensor | None = None) -> torch.Tensor:
    """Int8 GEMM with the fused epilogue: dequantize, + bias, ReLU, then fp32 /
    bf16 output, or (out_dtype "i8") the next linear's int8 codes for its
    smoothing factor next_s and static step next_scale [1]."""
    code, tdt = _OUT[out_dtype]
    md, wm = _mode(mode), _wmode(w_mode)
    M, N, K, y = _gemm_args(xq, x_scale, wq, w_scale, md, wm, code, tdt, y)
    _vec(bias, N, "bias", xq.device)
    _vec(next_s, N, "next_s", xq.device)
    _vec(next_scale, 1, "next_scale", xq.device)
    epi = SqEpilogue(_ptr(bias), _ptr(next_s), _ptr(next_scale), int(bool(relu)))
    _check(lib().sq_gemm_w8a8_ex(_ptr(xq), _ptr(x_scale), md, _ptr(wq), _ptr(w_scale),
                                 wm, M, N, K, ctypes.byref(epi), _ptr(y), code,
                                 _stream(xq.device)))
    return y


def _stride(t: torch.Tensor | None, per_entry: int) -> int:
    """Elements between batch entries of a contiguous [B, ...] tensor; 0 when a
    single entry is shared by every batch entry."""
    if t is None:
        return 0
    if t.dim() >= 1 and t.numel() == per_entry:
        return 0
    return per_entry


def sq_bmm_w8a8(xq: torch.Tensor, x_scale: torch.Tensor | None, wq: torch.Tensor,
                w_scale: torch.Tensor | None, mode="per_token", out_dtype: str = "bf16",
                y: torch.Tensor | None = None, w_mode="per_channel") -> torch.Tensor:
    """Batched int8 GEMM (the attention products): xq [B, M, K], wq [B, N, K]
    (or [N, K] shared), x_scale [B, M] / [B, 1] / [1], w_scale [B, N] / [B, 1] /
    [1]; returns y [B, M, N]."""
    for t, n in ((xq, "xq"), (wq, "wq")):
        if not t.is_cuda or not t.is_contiguous() or t.dim() not in (2, 3):
            raise ValueError(f"{n} must be a contiguous 2-D or 3-D GPU tensor")
    B = xq.shape[0] if xq.dim() == 3 else wq.shape[0]
    M, K = xq.shape[-2:]
    N, K2 = wq.shape[-2:]
    if K != K2:
        raise ValueError("xq and wq disagree on K")
    md, wm = _mode(mode), _wmode(w_mode)
    code, tdt = _OUT[out_dtype]
    if code == SQ_I8:
        raise ValueError("the batched product has no int8 output")
    if y is None:
        y = torch.empty((B, M, N), dtype=tdt, device=xq.device)
    elif y.dtype != tdt or not y.is_cuda or not y.is_contiguous() or y.numel() != B * M * N:
        raise ValueError(f"y must be a contiguous GPU tensor of {B}x{M}x{N} {tdt}")
    if wq.device != xq.device or y.device != xq.device:
        raise ValueError("xq, wq and y must be on one device")
    xs_n = M if md == SQ_PER_TOKEN else 1
    ws_n = N if wm == SQ_W_PER_CHANNEL else 1
    if code != SQ_I32:
        _vec(x_scale, (xs_n, B * xs_n), "x_scale", xq.device)
        _vec(w_scale, (ws_n, B * ws_n), "w_scale", xq.device)
    _check(lib().sq_bmm_w8a8(
        _ptr(xq), 0 if xq.dim() == 2 else M * K, _ptr(x_scale), _stride(x_scale, xs_n), md,
        _ptr(wq), 0 if wq.dim() == 2 else N * K, _ptr(w_scale), _stride(w_scale, ws_n), wm,
        B, M, N, K, _ptr(y), M * N, code, _stream(xq.device)))
    return y


# ---- robust calibration ---------------------------------------------------------

def _workspace(nbytes: int, device, workspace=None) -> torch.Tensor:
    if workspace is not None:
        if not workspace.is_cuda or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def sq_channel_quantile(x: torch.Tensor, q: float, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Per-channel nearest-rank q-quantile of |x[:, j]| (floored), fp32 [K]."""
    _dev2d(x, "x")
    T, K = x.shape
    nb = lib().sq_channel_quantile_workspace_size(K)
    ws = _workspace(nb, x.device, workspace)
    if out is None:
        out = torch.empty(K, dtype=torch.float32, device=x.device)
    else:
        _vec(out, K, "out", x.device)
    _check(lib().sq_channel_quantile(_ptr(x), _dt(x), T, K, float(q), _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(x.device)))
    return out


def sq_channel_quantile_noalloc(x: torch.Tensor, q: float, out: torch.Tensor) -> torch.Tensor:
    """sq_channel_quantile without a workspace (the library's own per-device
    scratch; K <= SQ_NOALLOC_MAX_K): for callers that cannot allocate, so the
    output ``out`` (fp32 [K]) is required."""
    _dev2d(x, "x")
    T, K = x.shape
    _vec(out, K, "out", x.device)
    _check(lib().sq_channel_quantile_noalloc(_ptr(x), _dt(x), T, K, float(q), _ptr(out),
                                             _stream(x.device)))
    return out


def sq_calibrate_stat(act_stat: torch.Tensor, w: torch.Tensor, alpha: float,
                      ln_gamma: torch.Tensor | None = None, ln_beta: torch.Tensor | None = None,
                      out: dict | None = None, w_mode="per_channel") -> dict:
    """sq_calibrate with a given activation statistic [K] in place of the peak:
    returns dict(a, s, wq, w_scale, static_scale, w_absmax[, ln_gamma_s, ln_beta_s])."""
    wm = _wmode(w_mode)
    _dev2d(w, "w")
    N, K = w.shape
    dev = w.device
    if act_stat.dim() != 1:
        raise ValueError("act_stat must be a float32 [K] tensor")
    _vec(act_stat, K, "act_stat", dev)
    _vec(ln_gamma, K, "ln_gamma", dev)
    _vec(ln_beta, K, "ln_beta", dev)
    o = dict(out or {})
    f32 = dict(dtype=torch.float32, device=dev)
    nws = N if wm == SQ_W_PER_CHANNEL else 1
    vecs = {"a": K, "s": K, "w_scale": nws, "static_scale": 1, "w_absmax": K}
    if ln_gamma is not None:
        vecs.update(ln_gamma_s=K, ln_beta_s=K)
    for k, n in vecs.items():
        if k in o:
            _vec(o[k], n, f"out[{k!r}]", dev)
        else:
            o[k] = torch.empty(n, **f32)
    if "wq" in o:
        _out2d(o["wq"], N, K, "out['wq']", dev, torch.int8)
    else:
        o["wq"] = torch.empty((N, K), dtype=torch.int8, device=dev)
    _check(lib().sq_calibrate_stat(
        _ptr(act_stat), _ptr(w), _dt(w), N, K, float(alpha), wm, _ptr(ln_gamma), _ptr(ln_beta),
        _ptr(o["s"]), _ptr(o["wq"]), _ptr(o["w_scale"]), _ptr(o["static_scale"]),
        _ptr(o.get("ln_gamma_s")), _ptr(o.get("ln_beta_s")), _ptr(o["a"]), _ptr(o["w_absmax"]),
        _stream(dev)))
    return o


def sq_clip_count(x: torch.Tensor, static_scale: torch.Tensor, s: torch.Tensor | None = None,
                  ln_gamma_s: torch.Tensor | None = None, ln_beta_s: torch.Tensor | None = None,
                  ln_eps: float = 1e-5, per_channel: bool = False):
    """Saturated elements of the static quantizer: (count int64 [1], per-channel
    int32 [K] or None)."""
    _dev2d(x, "x")
    M, K = x.shape
    _vec(static_scale, 1, "static_scale", x.device)
    _vec(s, K, "s", x.device)
    _vec(ln_gamma_s, K, "ln_gamma_s", x.device)
    _vec(ln_beta_s, K, "ln_beta_s", x.device)
    count = torch.empty(1, dtype=torch.int64, device=x.device)
    pc = torch.empty(K, dtype=torch.int32, device=x.device) if per_channel else None
    _check(lib().sq_clip_count(_ptr(x), _dt(x), M, K, _ptr(s), _ptr(ln_gamma_s), _ptr(ln_beta_s),
                               float(ln_eps), _ptr(static_scale), _ptr(count), _ptr(pc),
                               _stream(x.device)))
    return count, pc


def sq_alpha_search(x_cal: torch.Tensor, w: torch.Tensor, alphas, mode="per_token",
                    w_mode="per_channel", workspace: torch.Tensor | None = None):
    """Candidate alphas for one linear: (err fp64 [n], werr fp64 [n], best int32 [1])."""
    _dev2d(x_cal, "x_cal")
    _dev2d(w, "w")
    T, K = x_cal.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("x_cal and w disagree on K")
    if x_cal.device != w.device:
        raise ValueError("x_cal and w must be on one device")
    al = (ctypes.c_float * len(alphas))(*[float(a) for a in alphas])
    nb = lib().sq_alpha_search_workspace_size(T, N, K)
    ws = _workspace(nb, w.device, workspace)
    err = torch.empty(len(alphas), dtype=torch.float64, device=w.device)
    werr = torch.empty(len(alphas), dtype=torch.float64, device=w.device)
    best = torch.empty(1, dtype=torch.int32, device=w.device)
    _check(lib().sq_alpha_search(
        _ptr(x_cal), _dt(x_cal), T, _ptr(w), _dt(w), N, K, ctypes.addressof(al), len(alphas),
        _mode(mode), _wmode(w_mode), _ptr(err), _ptr(werr), _ptr(best), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(w.device)))
    return err, werr, best
