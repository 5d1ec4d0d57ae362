"""CPU oracle for the SmoothQuant W8A8 linear-layer path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does; the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp32 operations in a fixed
order, fp64 where stated).  This module only marshals numpy arrays through
ctypes and adds the fp64 reference products used by the identity and error
checks ([Review] §5.1 eq. (3): XW = (X diag(s)^-1)(diag(s)W) in exact
arithmetic).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32 = 0
BF16 = 1
FLOOR = np.float32(1e-7)

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no FMA contraction, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lquadmath", "-lm"]
    subprocess.check_call(cmd, cwd=_HERE)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, f32p, i8p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        ci, cf = ctypes.c_int, ctypes.c_float
        L.orc_colmax.argtypes = [vp, ci, i64, i64, f32p]
        L.orc_smooth_factor.argtypes = [f32p, f32p, i64, cf, f32p]
        L.orc_smooth_factor_audit.argtypes = [f32p, f32p, i64, cf, vp, vp]
        L.orc_weight_quant.argtypes = [vp, ci, i64, i64, f32p, vp, i64, i8p, f32p]
        L.orc_weight_quant_per_input.argtypes = [vp, ci, i64, i64, f32p, i8p, f32p]
        L.orc_ln_fold.argtypes = [f32p, f32p, f32p, i64, f32p, f32p]
        L.orc_static_scale.argtypes = [f32p, f32p, i64]
        L.orc_static_scale.restype = ctypes.c_float
        L.orc_act_smooth.argtypes = [vp, ci, i64, i64, f32p, vp, i64, f32p]
        L.orc_act_ln.argtypes = [vp, ci, i64, i64, f32p, f32p, cf, vp, i64, f32p]
        L.orc_canonical_sum.argtypes = [f32p, i64]
        L.orc_canonical_sum.restype = ctypes.c_float
        L.orc_quant_per_token.argtypes = [f32p, i64, i64, i8p, f32p]
        L.orc_quant_static.argtypes = [f32p, i64, i64, cf, i8p]
        L.orc_quant_static.restype = ctypes.c_int64
        L.orc_gemm_i32.argtypes = [i8p, i8p, i64, i64, i64, vp]
        L.orc_gemm_i32.restype = ci
        L.orc_dequant.argtypes = [vp, f32p, ci, f32p, ci, i64, i64, f32p]
        L.orc_epilogue.argtypes = [f32p, i64, i64, vp, ci, f32p]
        L.orc_requant.argtypes = [f32p, i64, i64, vp, cf, i8p]
        L.orc_requant.restype = ctypes.c_int64
        L.orc_weight_quant_per_tensor.argtypes = [vp, ci, i64, i64, f32p, i8p]
        L.orc_weight_quant_per_tensor.restype = ctypes.c_float
        L.orc_quant_dynamic_per_tensor.argtypes = [f32p, i64, i64, i8p]
        L.orc_quant_dynamic_per_tensor.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [f32p, i64, vp]
        L.orc_ln_f64.argtypes = [vp, ci, i64, i64, vp, vp, ctypes.c_double, vp]
        L.orc_num_threads.restype = ci
        L.orc_set_num_threads.argtypes = [ci]
        L.orc_set_num_threads.restype = None
        _lib = L
    return _lib


# ---- marshalling helpers ---------------------------------------------------

def _raw(x: np.ndarray):
    """(pointer, dtype code) of a C-contiguous fp32 or bf16-bits (uint16) array."""
    if x.dtype == np.float32:
        dt = F32
    elif x.dtype == np.uint16:
        dt = BF16
    else:
        raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {x.dtype}")
    if not x.flags.c_contiguous:
        raise ValueError("oracle input must be C-contiguous")
    return x.ctypes.data, dt


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def _rows(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.ctypes.data, int(r.size)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---- the path ----------------------------------------------------------------

def colmax(x: np.ndarray) -> np.ndarray:
    rows, K = x.shape
    p, dt = _raw(x)
    out = np.empty(K, np.float32)
    lib().orc_colmax(p, dt, rows, K, out.ctypes.data)
    return out


def smooth_factor(a, w, alpha: float) -> np.ndarray:
    a, w = _f32(a), _f32(w)
    s = np.empty(a.size, np.float32)
    lib().orc_smooth_factor(a.ctypes.data, w.ctypes.data, a.size, float(alpha), s.ctypes.data)
    return s


def smooth_factor_audit(a, w, alpha: float):
    """(near-tie channel count, fp64-vs-quad rounding mismatches)."""
    a, w = _f32(a), _f32(w)
    t = ctypes.c_int64(0)
    m = ctypes.c_int64(0)
    lib().orc_smooth_factor_audit(a.ctypes.data, w.ctypes.data, a.size, float(alpha),
                                  ctypes.addressof(t), ctypes.addressof(m))
    return int(t.value), int(m.value)


def weight_quant(w: np.ndarray, s, rows=None):
    N, K = w.shape
    p, dt = _raw(w)
    s = _f32(s)
    r, rp, nr = _rows(rows)
    n_out = N if r is None else nr
    wq = np.empty((n_out, K), np.int8)
    sc = np.empty(n_out, np.float32)
    lib().orc_weight_quant(p, dt, N, K, s.ctypes.data, rp, nr, wq.ctypes.data, sc.ctypes.data)
    return wq, sc


def weight_quant_per_tensor(w: np.ndarray, s):
    """Per-tensor weight step ([Review] §6.3, SmoothQuant-O1..O3): (codes, [dw])."""
    N, K = w.shape
    p, dt = _raw(w)
    s = _f32(s)
    wq = np.empty((N, K), np.int8)
    d = lib().orc_weight_quant_per_tensor(p, dt, N, K, s.ctypes.data, wq.ctypes.data)
    return wq, np.array([d], np.float32)


def weight_quant_per_input(w: np.ndarray, s):
    N, K = w.shape
    p, dt = _raw(w)
    s = _f32(s)
    wq = np.empty((N, K), np.int8)
    cs = np.empty(K, np.float32)
    lib().orc_weight_quant_per_input(p, dt, N, K, s.ctypes.data, wq.ctypes.data, cs.ctypes.data)
    return wq, cs


def ln_fold(gamma, beta, s):
    g, b, s = _f32(gamma), _f32(beta), _f32(s)
    gs = np.empty_like(g)
    bs = np.empty_like(b)
    lib().orc_ln_fold(g.ctypes.data, b.ctypes.data, s.ctypes.data, g.size,
                      gs.ctypes.data, bs.ctypes.data)
    return gs, bs


def static_scale(a, s) -> np.float32:
    a, s = _f32(a), _f32(s)
    return np.float32(lib().orc_static_scale(a.ctypes.data, s.ctypes.data, a.size))


def act_smooth(x: np.ndarray, s, rows=None) -> np.ndarray:
    M, K = x.shape
    p, dt = _raw(x)
    s = _f32(s)
    r, rp, nr = _rows(rows)
    out = np.empty((M if r is None else nr, K), np.float32)
    lib().orc_act_smooth(p, dt, M, K, s.ctypes.data, rp, nr, out.ctypes.data)
    return out


def act_ln(x: np.ndarray, g_s, b_s, eps: float = 1e-5, rows=None) -> np.ndarray:
    M, K = x.shape
    p, dt = _raw(x)
    g_s, b_s = _f32(g_s), _f32(b_s)
    r, rp, nr = _rows(rows)
    out = np.empty((M if r is None else nr, K), np.float32)
    lib().orc_act_ln(p, dt, M, K, g_s.ctypes.data, b_s.ctypes.data, float(eps), rp, nr,
                     out.ctypes.data)
    return out


def canonical_sum(v) -> np.float32:
    v = _f32(v)
    return np.float32(lib().orc_canonical_sum(v.ctypes.data, v.size))


def quant_per_token(xhat):
    xhat = _f32(xhat)
    M, K = xhat.shape
    q = np.empty((M, K), np.int8)
    sc = np.empty(M, np.float32)
    lib().orc_quant_per_token(xhat.ctypes.data, M, K, q.ctypes.data, sc.ctypes.data)
    return q, sc


def quant_dynamic_per_tensor(xhat):
    """Dynamic per-tensor activation step ([Review] §6.3, SmoothQuant-O2): (codes, [d])."""
    xhat = _f32(xhat)
    M, K = xhat.shape
    q = np.empty((M, K), np.int8)
    d = lib().orc_quant_dynamic_per_tensor(xhat.ctypes.data, M, K, q.ctypes.data)
    return q, np.array([d], np.float32)


def quant_static(xhat, scale):
    xhat = _f32(xhat)
    M, K = xhat.shape
    q = np.empty((M, K), np.int8)
    sat = lib().orc_quant_static(xhat.ctypes.data, M, K, float(np.float32(scale)), q.ctypes.data)
    return q, int(sat)


def gemm_i32(xq, wq) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("contraction sizes differ")
    acc = np.empty((M, N), np.int32)
    rc = lib().orc_gemm_i32(xq.ctypes.data, wq.ctypes.data, M, N, K, acc.ctypes.data)
    if rc != 0:
        raise OverflowError("int8 GEMM accumulator exceeds int32")
    return acc


def dequant(acc, x_scale, w_scale, per_token: bool = True,
            w_per_tensor: bool = False) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    xs, ws = _f32(x_scale), _f32(w_scale)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    lib().orc_dequant(acc.ctypes.data, xs.ctypes.data, int(bool(per_token)), ws.ctypes.data,
                      int(bool(w_per_tensor)), M, N, y.ctypes.data)
    return y


def epilogue(y, bias=None, relu=False) -> np.ndarray:
    """Bias (one RN addition) then ReLU (y > 0 ? y : +0) on fp32 outputs."""
    y = _f32(y)
    M, N = y.shape
    b = None if bias is None else _f32(bias)
    out = np.empty_like(y)
    lib().orc_epilogue(y.ctypes.data, M, N, None if b is None else b.ctypes.data, int(bool(relu)),
                       out.ctypes.data)
    return out


def requant(y, next_s, step):
    """int8 codes of y for the next linear (smoothing s', static step): (codes, n_saturated)."""
    y = _f32(y)
    M, N = y.shape
    ns = None if next_s is None else _f32(next_s)
    q = np.empty((M, N), np.int8)
    sat = lib().orc_requant(y.ctypes.data, M, N, None if ns is None else ns.ctypes.data,
                            float(np.float32(step)), q.ctypes.data)
    return q, int(sat)


def f32_to_bf16(y) -> np.ndarray:
    y = _f32(y)
    out = np.empty(y.shape, np.uint16)
    lib().orc_f32_to_bf16(y.ctypes.data, y.size, out.ctypes.data)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ln_f64(x, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    M, K = x.shape
    p, dt = _raw(x)
    g = np.ascontiguousarray(gamma, dtype=np.float64)
    b = np.ascontiguousarray(beta, dtype=np.float64)
    out = np.empty((M, K), np.float64)
    lib().orc_ln_f64(p, dt, M, K, g.ctypes.data, b.ctypes.data, float(eps), out.ctypes.data)
    return out


def as_f64(x: np.ndarray) -> np.ndarray:
    """fp64 view of a raw input (fp32 or bf16 bits)."""
    if x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def ref_linear_f64(x, w) -> np.ndarray:
    """Y64 = X W^T in fp64 (W stored [out, in])."""
    return as_f64(x) @ as_f64(w).T


def ref_smoothed_linear_f64(x, w, s) -> np.ndarray:
    """Yhat64 = (X diag(s)^-1)(diag(s) W) in fp64 -- [Review] §5.1 eq. (3)."""
    s64 = np.asarray(s, dtype=np.float64)
    return (as_f64(x) / s64[None, :]) @ (as_f64(w) * s64[None, :]).T


# ---- whole-path composition (oracle side) ------------------------------------

def calibrate(x_cal, w, alpha, gamma=None, beta=None, rows=None, w_per_tensor=False,
              act_stat=None):
    """Offline half: colmax of X_cal and W, eq. (4), smoothed int8 weights
    (per output channel, or per tensor for the [Review] §6.3 O1-O3 settings),
    optional LayerNorm fold and the static activation scale.  act_stat [K]:
    a per-channel activation statistic used in place of the calibration peak
    (floored like the peak; [Teach] §四 allows a robust statistic), x_cal is
    then not read."""
    if act_stat is not None:
        a = np.maximum(_f32(act_stat), FLOOR)
    else:
        a = colmax(x_cal)
    wm = colmax(w)
    s = smooth_factor(a, wm, alpha)
    if w_per_tensor:
        if rows is not None:
            raise ValueError("a per-tensor weight step needs every row")
        wq, w_scale = weight_quant_per_tensor(w, s)
    else:
        wq, w_scale = weight_quant(w, s, rows=rows)
    out = dict(a=a, wmax=wm, s=s, wq=wq, w_scale=w_scale, static_scale=static_scale(a, s))
    if gamma is not None:
        out["g_s"], out["b_s"] = ln_fold(gamma, beta, s)
    return out


def smooth_quantize_act(x, s=None, g_s=None, b_s=None, eps=1e-5, static=None, rows=None,
                        dynamic_per_tensor=False):
    """Runtime half on the activation side; returns (codes, scales, n_saturated).
    dynamic_per_tensor: one step over the whole batch ([Review] §6.3 O2)."""
    if s is not None:
        xhat = act_smooth(x, s, rows=rows)
    else:
        xhat = act_ln(x, g_s, b_s, eps=eps, rows=rows)
    if dynamic_per_tensor:
        if rows is not None:
            raise ValueError("a per-tensor step needs every token")
        q, d = quant_dynamic_per_tensor(xhat)
        return q, d, 0
    if static is None:
        q, sc = quant_per_token(xhat)
        return q, sc, 0
    q, sat = quant_static(xhat, static)
    return q, np.array([static], np.float32), sat


def gemm_w8a8(xq, x_scale, wq, w_scale, per_token=True, out="f32", w_per_tensor=False,
              bias=None, relu=False, next_s=None, next_scale=None):
    """Int8 GEMM, dequantization, then the optional fused epilogue; out "i8"
    requantizes for the next linear (next_s, next_scale)."""
    acc = gemm_i32(xq, wq)
    if out == "i32":
        return acc
    y = dequant(acc, x_scale, w_scale, per_token=per_token, w_per_tensor=w_per_tensor)
    if bias is not None or relu:
        y = epilogue(y, bias, relu)
    if out == "i8":
        return requant(y, next_s, next_scale)[0]
    if out == "bf16":
        return f32_to_bf16(y)
    return y


def bmm_w8a8(xq, x_scale, wq, w_scale, per_token=True, w_per_tensor=False, out="f32"):
    """Batched int8 GEMM ([Review] §5.6, Fig. 6: the batched matrix products of
    attention run in int8 like the linear layers): entry b is gemm_w8a8 of
    xq[b] [M, K] with wq[b] [N, K] and the b-th scale vectors."""
    B = xq.shape[0]
    outs = [gemm_w8a8(xq[b], x_scale[b], wq[b], w_scale[b], per_token=per_token, out=out,
                      w_per_tensor=w_per_tensor) for b in range(B)]
    return np.stack(outs)


# ---- robust calibration ([Teach] §四, §六, §八) ---------------------------------

def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_to_f32(x) if x.dtype == np.uint16 else np.ascontiguousarray(x, np.float32)


def quantile_rank(T: int, q) -> int:
    """1-based nearest rank of the q-quantile among T values: ceil(q T) in fp64,
    at least 1 and at most T."""
    import math
    return max(1, min(int(T), math.ceil(float(np.float32(q)) * float(T))))


def channel_quantile(x, q) -> np.ndarray:
    """Robust per-channel activation statistic ([Teach] §四: the calibration may
    record a robust statistic instead of the peak): for channel j the
    nearest-rank q-quantile of |x[:, j]|, i.e. the quantile_rank(T, q)-th
    smallest magnitude, floored at FLOOR.  q = 1 is the peak of a1."""
    xa = np.abs(_as_f32(x))
    T, K = xa.shape
    if T == 0:
        return np.full(K, FLOOR, np.float32)
    v = np.sort(xa, axis=0)[quantile_rank(T, q) - 1]
    return np.maximum(v, FLOOR).astype(np.float32)


def clip_counts(xhat, scale):
    """Saturation of the static quantizer ([Teach] §六: check the clip rate per
    layer): codes whose rounded quotient rne(RN(xhat / scale)) lies outside
    [-127, 127].  Returns (total, per-channel counts [K])."""
    xh = _f32(xhat)
    q = np.rint(xh / np.float32(scale))
    c = np.abs(q) > 127
    return int(c.sum()), c.sum(axis=0).astype(np.int64)


def _rel(num: float, den: float) -> float:
    return num / den if den > 0 else num


def alpha_search(x_cal, w, alphas, mode="per_token", w_per_tensor=False):
    """Candidate alphas for one linear ([Teach] §八: on candidate alphas measure
    activation saturation, weight quantization error and the task set, per
    layer if needed).  For each alpha, on the calibration batch:
      err  = sum (y_q - y)^2 / sum y^2, y_q the dequantized fp32 output of the
             quantized linear (activation mode as deployed), y = X W^T in fp64
             (stands in for the task-set check, which needs a trained model);
      werr = sum (W^ - dw q)^2 / sum W^^2 over the smoothed weights W^ = RN(W s)
             and their dequantized codes (in fp64).
    A ratio with a zero denominator is its numerator.  best = the first alpha
    of least err.  The saturation check is clip_counts on held-out tokens."""
    y64 = ref_linear_f64(x_cal, w)
    den = float((y64 * y64).sum())
    wf = _as_f32(w)
    errs, werrs = [], []
    for al in alphas:
        cal = calibrate(x_cal, w, float(np.float32(al)), w_per_tensor=w_per_tensor)
        static = cal["static_scale"] if mode == "static" else None
        xq, xs, _ = smooth_quantize_act(x_cal, s=cal["s"], static=static,
                                        dynamic_per_tensor=mode == "dynamic_per_tensor")
        yq = gemm_w8a8(xq, xs, cal["wq"], cal["w_scale"], per_token=mode == "per_token",
                       out="f32", w_per_tensor=w_per_tensor)
        d = yq.astype(np.float64) - y64
        errs.append(_rel(float((d * d).sum()), den))
        what = (wf * cal["s"][None, :]).astype(np.float64)          # RN(W s) in fp32
        ws = np.broadcast_to(cal["w_scale"].astype(np.float64)[:, None]
                             if not w_per_tensor else cal["w_scale"].astype(np.float64)[0],
                             what.shape)
        dw = what - cal["wq"].astype(np.float64) * ws
        werrs.append(_rel(float((dw * dw).sum()), float((what * what).sum())))
    return np.array(errs), np.array(werrs), int(np.argmin(errs))
