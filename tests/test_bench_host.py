"""Host-side checks of bench.py that need no GPU: the single-GPU contract
(any --gpus other than 1 exits with status 2 and says why, before touching a
device) and the workload table."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_workloads_listed():
    sys.path.insert(0, ROOT)
    import bench
    assert {"opt6.7b", "attn6.7b", "robust8192", "decode70b", "opt175b", "ln8192"} <= set(bench.WORKLOADS)


def test_alpha_sweep_spread_closed_forms():
    """The alpha sweep's spread ([Review] §5.3 eq. (4)): with s from the oracle's
    calibration of the LayerNorm workload, the smoothed activation peaks are
    a_j / s_j = (a_j w_j)^(1 - alpha) and the weight peaks w_j s_j =
    (a_j w_j)^alpha, so with R = max(a w) / min(a w) the activation spread is
    R^(1 - alpha) and the weight spread R^alpha (to fp32 rounding); alpha = 1
    makes every smoothed activation peak exactly 1 (spread 1, bit for bit)."""
    sys.path.insert(0, ROOT)
    import numpy as np

    import bench
    import datagen
    import oracle

    spec = datagen.workload(5).layers[0]
    xc = datagen.calibration_x(spec, T=1024)
    w = datagen.weights(spec)[:512]
    g, b = datagen.ln_params(spec)
    a = oracle.colmax(xc)
    wm = oracle.colmax(w)
    R = float((a.astype(np.float64) * wm).max() / (a.astype(np.float64) * wm).min())
    assert R > 100  # outlier channels make the raw spread large
    for alpha in (0.0, 0.25, 0.5, 0.75, 0.85, 1.0):
        cal = oracle.calibrate(xc, w, alpha, g, b)
        sa = bench.smoothed_spread(cal["a"], cal["s"])
        sw = bench.smoothed_spread(cal["wmax"], cal["s"], weight=True)
        assert abs(np.log(sa) - (1 - alpha) * np.log(R)) < 1e-5
        assert abs(np.log(sw) - alpha * np.log(R)) < 1e-5
        if alpha == 1.0:
            assert sa == 1.0
        if alpha == 0.0:
            assert abs(sw - 1.0) < 3e-7


def test_alpha_sweep_fp64_reference_matches_the_oracle():
    """bench.py's fp64 LayerNorm-linear reference equals the oracle's pinned
    fp64 LayerNorm times W^T (to fp64 rounding)."""
    sys.path.insert(0, ROOT)
    import numpy as np

    import bench
    import datagen
    import oracle

    spec = datagen.workload(5).layers[0]
    x = datagen.eval_x(spec, M=16)
    w = datagen.weights(spec)[:300]
    g, b = datagen.ln_params(spec)
    ref = oracle.ln_f64(x, g.astype(np.float64), b.astype(np.float64), 1e-5) @ \
        oracle.as_f64(w).T
    got = bench.ln_linear_f64(datagen.bf16_bits_to_f32(x), g, b, datagen.bf16_bits_to_f32(w))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_alpha_sweep_needs_the_layernorm_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--alpha-sweep"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "ln8192" in r.stderr
