"""Seeded randomized shapes through the whole path (calibrate, quantize, int8
GEMM), every element against the oracle: sizes drawn across every kernel's
range (decode M <= 64, short K of 64 / 128 / 256, the ping-pong tiles, K not a
multiple of 128, ragged M and N down to 1, rows up to 49152 elements), with
random input dtypes, step granularities, weight modes, LayerNorm fold and
alpha.  The case lists are fixed by their seeds, so a failure names a
reproducible case.
"""
import numpy as np
import pytest

import datagen
from sqcase import run_layer

pytestmark = pytest.mark.gpu

_KS = [64, 128, 192, 256, 320, 384, 448, 512, 640, 768, 1024, 1152, 1536]


def _cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        small_m = rng.random() < 0.3
        M = int(rng.integers(1, 65)) if small_m else int(rng.integers(65, 601))
        N = int(rng.integers(1, 1201))
        K = int(rng.choice(_KS))
        xdt = str(rng.choice(["bf16", "f32"]))
        wdt = str(rng.choice(["bf16", "f32"]))
        mode = str(rng.choice(["per_token", "static", "dynamic_per_tensor"]))
        wmode = str(rng.choice(["per_channel", "per_tensor"]))
        ln = bool(rng.random() < 0.3)
        alpha = float(rng.choice(datagen.ALPHA_SWEEP))
        out.append((i, M, N, K, xdt, wdt, mode, wmode, ln, alpha))
    return out


CASES = _cases()

# long rows: every kernel range of the quantizers and the weight path (one-row,
# two-row, recomputing and per-tensor streaming kernels), smaller M and N
_KS_LONG = [2048, 2112, 4160, 6144, 8256, 12288, 16384, 16448, 24576, 36928, 49152]


def _cases_long(n=40, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(rng.choice(_KS_LONG))
        M = int(rng.integers(1, 48))
        N = int(rng.integers(1, 260))
        xdt = str(rng.choice(["bf16", "bf16", "f32"]))
        wdt = str(rng.choice(["bf16", "bf16", "f32"]))
        mode = str(rng.choice(["per_token", "static", "dynamic_per_tensor"]))
        wmode = str(rng.choice(["per_channel", "per_tensor"]))
        ln = bool(rng.random() < 0.3) and K <= 16448
        alpha = float(rng.choice(datagen.ALPHA_SWEEP))
        out.append((100 + i, M, N, K, xdt, wdt, mode, wmode, ln, alpha))
    return out


CASES += _cases_long()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"r{c[0]}_{c[1]}x{c[2]}x{c[3]}_{c[4]}_{c[5]}_"
                         f"{c[6]}_{c[7]}_{'ln' if c[8] else 'plain'}_a{c[9]}")
def test_random_shape_every_element(case):
    i, M, N, K, xdt, wdt, mode, wmode, ln, alpha = case
    spec = datagen.random_layer(M, N, K, seed=7000 + 13 * i, x_dtype=xdt, w_dtype=wdt,
                                n_outliers=max(1, K // 128), T=max(8, min(M, 64)), alpha=alpha,
                                mode=mode, ln=ln)
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    g = b = None
    if ln:
        g, b = datagen.ln_params(spec)
    run_layer(spec, xc, w, x, mode, gamma=g, beta=b, alpha=alpha, w_mode=wmode)
