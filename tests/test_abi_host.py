"""Host-side checks of libsq.so that need no GPU: the library loads, exports
every entry point include/sq.h declares, and rejects invalid arguments with the
documented status before touching the device (so only fake, never-dereferenced
pointers are passed here, and only to calls that must fail validation)."""
import ctypes
import os
import re
import subprocess

import pytest

import w8a8_int8_gemm_colwise_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sq.h")

P = 0x1000      # aligned fake device pointer (never dereferenced: validation fails first)
MIS = 0x1008    # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sq_status|const char\s*\*|int|size_t)\s+(sq_\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_version():
    L = sq.lib()
    assert L.sq_abi_version() == sq.SQ_ABI_VERSION


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"sq_calibrate", "sq_smooth_quantize_act", "sq_gemm_w8a8",
                          "sq_status_string", "sq_abi_version"}
    L = sq.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (sq_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    assert set(sq.EXPORTED) <= exported


def test_status_strings():
    L = sq.lib()
    for code in range(9):
        s = L.sq_status_string(code).decode()
        assert s.startswith("SQ_")
    assert L.sq_status_string(99).decode() == "SQ_ERR_UNKNOWN"


def _gemm(M=4, N=4, K=64, xq=P, xs=P, mode=0, wq=P, ws=P, wmode=0, y=P, ydt=0):
    return sq.lib().sq_gemm_w8a8(xq, xs, mode, wq, ws, wmode, M, N, K, y, ydt, None)


def _act(M=4, K=64, x=P, dt=1, s=P, g=None, b=None, eps=1e-5, mode=0, st=None, xq=P, xs=P):
    return sq.lib().sq_smooth_quantize_act(x, dt, M, K, s, g, b, eps, mode, st, xq, xs, None)


def _cal(T=8, N=8, K=64, alpha=0.5, xdt=1, wdt=1, g=None, b=None, gs=None, bs=None, x=P, w=P,
         s=P, wq=P, wsc=P, st=P, xa=P, wa=P, wmode=0):
    return sq.lib().sq_calibrate(x, xdt, T, w, wdt, N, K, alpha, wmode, g, b, s, wq, wsc, st, gs,
                                 bs, xa, wa, None)


@pytest.mark.parametrize("K", [0, -64, 63, 65, 100, sq.SQ_MAX_K + 64])
def test_gemm_rejects_bad_k(K):
    assert _gemm(K=K) == 2


def test_gemm_validation():
    assert _gemm(M=-1) == 2
    assert _gemm(N=-1) == 2
    assert _gemm(ydt=7) == 3
    assert _gemm(ydt=2) == 3          # int8 output is not an output type
    assert _gemm(mode=5) == 7
    assert _gemm(wmode=2) == 7
    assert _gemm(wmode=-1) == 7
    assert _gemm(xq=None) == 1
    assert _gemm(wq=None) == 1
    assert _gemm(y=None) == 1
    assert _gemm(xs=None) == 1        # dequant needs scales
    assert _gemm(ws=None) == 1
    assert _gemm(xq=MIS) == 5
    assert _gemm(y=MIS) == 5
    # M = 0 or N = 0: nothing to do, succeeds without touching the device
    assert _gemm(M=0, xq=None, y=None) == 0
    assert _gemm(N=0, wq=None, y=None) == 0


def test_act_validation():
    assert _act(K=96) == 2
    assert _act(M=-3) == 2
    assert _act(dt=2) == 3
    assert _act(mode=3) == 7
    assert _act(mode=2, xs=None) == 1                  # dynamic per-tensor writes its step
    assert _act(s=None) == 1                           # neither plain nor LN
    assert _act(g=P, b=P) == 7                         # both plain and LN
    assert _act(s=None, g=P, b=None) == 1              # half of LN
    assert _act(s=None, g=P, b=P, eps=0.0) == 7
    assert _act(s=None, g=P, b=P, eps=float("nan")) == 7
    assert _act(mode=1, st=None) == 1                  # static mode needs the scale
    assert _act(xs=None) == 1                          # per-token mode writes scales
    assert _act(x=MIS) == 5
    assert _act(xq=MIS) == 5
    assert _act(M=0, x=None, xq=None, xs=None) == 0
    # an empty batch in dynamic per-tensor mode still writes its step
    # (FLOOR / 127) into x_scale[0]: a missing x_scale is rejected on the host
    assert _act(M=0, mode=2, x=None, xq=None, xs=None) == 1


def test_calibrate_validation():
    assert _cal(K=32) == 2
    assert _cal(T=-1) == 2
    assert _cal(N=-1) == 2
    assert _cal(xdt=3) == 3
    assert _cal(wdt=2) == 3
    for a in (-0.01, 1.01, float("nan"), float("inf")):
        assert _cal(alpha=a) == 4
    assert _cal(s=None) == 1
    assert _cal(xa=None) == 1
    assert _cal(wa=None) == 1
    assert _cal(x=None) == 1
    assert _cal(wq=None) == 1
    assert _cal(g=P, b=None) == 7                      # gamma without beta
    assert _cal(g=P, b=P, gs=None, bs=P) == 1          # fold outputs required
    assert _cal(wsc=MIS) == 5
    assert _cal(wmode=2) == 7
    assert _cal(wmode=1, wsc=None) == 1                # the per-tensor step is an output
    assert _cal(wmode=1, N=0, w=None, wq=None, wsc=None) == 1


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sq.sq_smooth_quantize_act(x, s=torch.ones(64))


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(sq, "_lib", None)
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "libsq.so"))
    with pytest.raises(RuntimeError):
        sq.lib()


def test_library_has_no_unresolved_kernel_stubs():
    """Every kernel launch in the library resolves to a kernel stub in the same
    library (a template kernel whose host stub the compiler failed to emit
    would leave an undefined symbol that only shows at load time)."""
    import shutil
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", sq.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert "__device_stub" not in out


def test_probe_library_exports_and_validates():
    """libsqprobe.so (the benchmark's attainable-ceiling probes) exports what
    include/sq_probe.h declares and rejects invalid arguments before launching."""
    from w8a8_int8_gemm_colwise_amd import probes
    text = open(os.path.join(ROOT, "include", "sq_probe.h")).read()
    names = set(re.findall(r"^\s*int\s+(sqp_\w+)\s*\(", text, flags=re.M))
    assert names == {"sqp_mfma_i8", "sqp_read", "sqp_copy", "sqp_check_rcp",
                     "sqp_check_div_narrow", "sqp_check_div", "sqp_check_codes", "sqp_div_ref"}
    out = subprocess.run(["nm", "-D", "--defined-only", probes.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert names <= set(re.findall(r" T (sqp_\w+)$", out, flags=re.M))
    L = probes.lib()
    assert L.sqp_mfma_i8(None, 4, 8, P, None) == 1
    assert L.sqp_mfma_i8(P, 4, 12, P, None) == 1          # iters not a multiple of 8
    assert L.sqp_read(P, 100, 4, P, None) == 1            # bytes not a multiple of 16
    assert L.sqp_read(MIS, 64, 4, P, None) == 1           # misaligned
    assert L.sqp_copy(P, MIS, 64, 4, None) == 1
    assert L.sqp_copy(P, P + 64, 0, 4, None) == 1
    assert L.sqp_check_rcp(0x3F800000, 0x40000000, 0, None, P, None) == 1
    assert L.sqp_check_rcp(0x40000000, 0x3F800000, 0, P, P, None) == 1   # empty range
    assert L.sqp_check_rcp(0x00400000, 0x3F800000, 0, P, P, None) == 1   # subnormal b
    assert L.sqp_check_rcp(0x3F800000, 0x7F800001, 0, P, P, None) == 1   # past +inf
    assert L.sqp_check_div_narrow(0, P, None, None) == 1
    assert L.sqp_check_div(1, 0, 0, P, P, None) == 1
    assert L.sqp_check_codes(1, 0, 0, 0, P, P, None) == 1
    assert L.sqp_check_codes(1, 4, 1, 0, None, P, None) == 1
    assert L.sqp_div_ref(P, P, P, 0, None) == 1


def _gemm_ex(epi, ydt=0, **kw):
    a = dict(M=4, N=4, K=64, xq=P, xs=P, mode=0, wq=P, ws=P, wmode=0, y=P)
    a.update(kw)
    e = None if epi is None else sq.SqEpilogue(*epi)
    return sq.lib().sq_gemm_w8a8_ex(a["xq"], a["xs"], a["mode"], a["wq"], a["ws"], a["wmode"],
                                    a["M"], a["N"], a["K"], e, a["y"], ydt, None)


def test_gemm_ex_validation():
    """The fused epilogue: int8 output needs the next layer's step; next_s only
    with int8 output; raw int32 output takes no epilogue; pointers aligned."""
    assert _gemm_ex((None, None, None, 0), ydt=2) == 1          # i8 without next_scale
    assert _gemm_ex((None, P, None, 0), ydt=2) == 1
    assert _gemm_ex((None, P, P, 0), ydt=1) == 7                # next_s with bf16 output
    assert _gemm_ex((None, None, P, 0), ydt=0) == 7             # next_scale with f32 output
    assert _gemm_ex((P, None, None, 0), ydt=3) == 7             # bias with int32 output
    assert _gemm_ex((None, None, None, 1), ydt=3) == 7          # relu with int32 output
    assert _gemm_ex((MIS, None, None, 0), ydt=0) == 5
    assert _gemm_ex((None, MIS, P, 0), ydt=2) == 5
    assert _gemm_ex(None, ydt=9) == 3
    assert _gemm_ex(None, ydt=0, K=96) == 2
    assert _gemm_ex((P, None, None, 1), ydt=0, M=0, xq=None, y=None) == 0
    # the plain entry point has no int8 output
    assert _gemm(ydt=2) == 3


def _bmm(batch=2, M=4, N=4, K=64, xq=P, xqs=64 * 4, xs=P, xss=4, mode=0, wq=P, wqs=64 * 4,
         ws=P, wss=4, wmode=0, y=P, ys=16, ydt=0):
    return sq.lib().sq_bmm_w8a8(xq, xqs, xs, xss, mode, wq, wqs, ws, wss, wmode, batch, M, N, K,
                                y, ys, ydt, None)


def test_bmm_validation():
    assert _bmm(batch=-1) == 2
    assert _bmm(batch=65536) == 2
    assert _bmm(K=96) == 2
    assert _bmm(xqs=-16) == 2
    assert _bmm(ydt=2) == 3               # no int8 output
    assert _bmm(mode=4) == 7
    assert _bmm(wmode=3) == 7
    assert _bmm(xq=None) == 1
    assert _bmm(ws=None) == 1
    assert _bmm(xqs=8) == 5               # entry bases must stay 16-byte aligned
    assert _bmm(wqs=24) == 5
    assert _bmm(y=MIS) == 5
    assert _bmm(batch=0, xq=None, wq=None, y=None) == 0


def test_noalloc_quantile_validation():
    """sq_channel_quantile_noalloc rejects K above SQ_NOALLOC_MAX_K, a missing
    or misaligned pointer and q outside (0, 1] before any launch."""
    L = sq.lib()
    f = lambda T=8, K=64, x=P, dt=1, q=0.5, out=P: L.sq_channel_quantile_noalloc(
        x, dt, T, K, q, out, None)
    assert f(K=sq.SQ_NOALLOC_MAX_K + 64) == 2
    assert f(K=96) == 2
    assert f(T=-1) == 2
    assert f(dt=2) == 3
    assert f(q=0.0) == 7
    assert f(q=1.5) == 7
    assert f(out=None) == 1
    assert f(x=None) == 1
    assert f(x=MIS) == 5
    assert f(out=MIS) == 5


def test_robust_calibration_validation():
    """Channel quantile, calibration from a statistic, clip count and alpha
    search reject bad arguments (and a short workspace) before any device work."""
    L = sq.lib()
    nq = L.sq_channel_quantile_workspace_size(64)
    assert nq >= 64 * 1024 and L.sq_channel_quantile_workspace_size(96) == 0

    def q(x=P, dt=1, T=4, K=64, qq=0.5, out=P, ws=P, nb=nq):
        return L.sq_channel_quantile(x, dt, T, K, qq, out, ws, nb, None)
    assert q(qq=0.0) == 7 and q(qq=1.5) == 7 and q(qq=float("nan")) == 7
    assert q(K=96) == 2 and q(T=-1) == 2 and q(dt=2) == 3
    assert q(out=None) == 1 and q(ws=None) == 1 and q(x=None) == 1
    assert q(x=MIS) == 5 and q(ws=MIS) == 5
    assert q(nb=nq - 1) == 8

    def cs(a=P, w=P, dt=1, N=4, K=64, alpha=0.5, wmode=0, g=None, b=None, s=P, wq=P, ws=P,
           st=P, gs=None, bs=None, ao=P, wa=P):
        return L.sq_calibrate_stat(a, w, dt, N, K, alpha, wmode, g, b, s, wq, ws, st, gs, bs, ao,
                                   wa, None)
    assert cs(a=None) == 1 and cs(ao=None) == 1 and cs(wq=None) == 1
    assert cs(alpha=1.5) == 4 and cs(wmode=5) == 7 and cs(K=96) == 2 and cs(dt=3) == 3
    assert cs(g=P) == 7 and cs(g=P, b=P) == 1 and cs(a=MIS) == 5

    def c(x=P, dt=1, M=4, K=64, s=P, g=None, b=None, eps=1e-5, st=P, cnt=P, pc=None):
        return L.sq_clip_count(x, dt, M, K, s, g, b, eps, st, cnt, pc, None)
    assert c(st=None) == 1 and c(cnt=None) == 1 and c(s=None) == 1
    assert c(g=P, b=P) == 7 and c(s=None, g=P) == 1 and c(s=None, g=P, b=P, eps=0.0) == 7
    assert c(K=96) == 2 and c(dt=2) == 3 and c(pc=MIS) == 5 and c(cnt=MIS) == 5

    na = L.sq_alpha_search_workspace_size(4, 4, 64)
    assert na > 0 and L.sq_alpha_search_workspace_size(4, 4, 96) == 0
    good = (ctypes.c_float * 2)(0.5, 0.25)
    bad = (ctypes.c_float * 2)(0.5, 1.5)

    def a(x=P, xdt=1, T=4, w=P, wdt=1, N=4, K=64, al=good, n=2, mode=0, wmode=0, err=P, werr=P,
          best=P, ws=P, nb=na):
        return L.sq_alpha_search(x, xdt, T, w, wdt, N, K, ctypes.addressof(al), n, mode, wmode,
                                 err, werr, best, ws, nb, None)
    assert a(n=0) == 2 and a(n=1025) == 2 and a(T=0) == 2 and a(K=96) == 2
    assert a(al=bad) == 4 and a(mode=3) == 7 and a(wmode=2) == 7 and a(xdt=2) == 3
    assert a(err=None) == 1 and a(best=None) == 1 and a(ws=None) == 1
    assert a(err=MIS) == 5 and a(nb=na - 1) == 8
