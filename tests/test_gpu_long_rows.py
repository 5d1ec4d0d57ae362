"""Per-token quantizer on long plain rows (2049-6144 sixteen-byte chunks, the
one-row-per-block kernel with the row's factors requested at the start of
each row) against the oracle, every element: four and six chunks per lane,
lane counts that leave copies of the row's last chunk in the tail lanes,
more tokens than blocks, bf16 and fp32 inputs, and factors outside
[2^-126, 2^126), where the reciprocal of s_k is the IEEE division.  Codes and
per-token steps must match bit for bit.
"""
import numpy as np
import pytest

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu

# (M, K, x dtype): K / 8 chunks; four chunks per lane up to 4096 chunks, six
# beyond
CASES = [
    (1, 16448, "bf16"),     # 2056 chunks, 576 lanes: 248 tail lanes
    (300, 24576, "bf16"),   # 3072 chunks, 768 lanes; 300 tokens over 256 blocks
    (257, 32768, "bf16"),   # 4096 chunks, 1024 lanes
    (5, 32832, "bf16"),     # 4104 chunks, six per lane, 704 lanes
    (513, 36928, "bf16"),   # 4616 chunks, 832 lanes, two sweeps of the grid
    (64, 49152, "bf16"),    # 6144 chunks, 1024 lanes
    (3, 49088, "bf16"),     # 6136 chunks: eight tail lanes in the last chunk
    (40, 24576, "f32"),
    (9, 32768, "f32"),
    (3, 49152, "f32"),      # six fp32 chunks per lane
]


def _inputs(M, K, xdt, seed):
    spec = datagen.random_layer(M, 8, K, seed=seed, x_dtype=xdt, n_outliers=max(1, K // 512),
                                T=16)
    x = datagen.eval_x(spec)
    a = oracle.colmax(datagen.calibration_x(spec))
    s = oracle.smooth_factor(a, oracle.colmax(datagen.weights(spec)), 0.5)
    return x, s


def _check(x, s):
    d = dev()
    xq_t, xs_t = sq.sq_smooth_quantize_act(to_dev(x, d), to_dev(s, d), mode="per_token")
    q_ref, sc_ref, _ = oracle.smooth_quantize_act(x, s=s)
    assert_same("xq", to_np(xq_t), q_ref)
    assert_same("x_scale", to_np(xs_t), sc_ref)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}")
def test_long_row_per_token_every_element(case):
    M, K, xdt = case
    say(f"[case] long-row per-token quantizer M={M} K={K} {xdt}")
    x, s = _inputs(M, K, xdt, 9500 + K + M)
    _check(x, s)


@pytest.mark.parametrize("K", [32832, 49152])
def test_long_row_factor_outside_fast_reciprocal_range(K):
    # one factor at 2^126 or above: the block takes the IEEE reciprocal path
    say(f"[case] long-row per-token quantizer, factor >= 2^126, K={K}")
    x, s = _inputs(17, K, "bf16", 9600 + K)
    s = s.copy()
    s[K // 3] = np.float32(1e38)
    assert s[K // 3] >= np.float32(2.0 ** 126)
    _check(x, s)
