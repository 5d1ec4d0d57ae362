"""A step of the path captured as a HIP graph and replayed: every replay
writes exactly what the eager calls write (calibration outputs, codes, steps,
GEMM output), with eager library work and synchronizations between the
replays; outputs are cleared before each replay so a replay that wrote
nothing would fail."""
import numpy as np
import pytest
import torch

import datagen
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import dev, say, to_dev

pytestmark = pytest.mark.gpu


def _layer(d, M, N, K, seed):
    spec = datagen.random_layer(M, N, K, seed=seed, n_outliers=3, T=128)
    xc, w, x = datagen.calibration_x(spec), datagen.weights(spec), datagen.eval_x(spec)
    f32 = dict(dtype=torch.float32, device=d)
    L = dict(xc=to_dev(xc, d), w=to_dev(w, d), x=to_dev(x, d), alpha=spec.alpha)
    L["cal"] = dict(s=torch.empty(K, **f32), wq=torch.empty((N, K), dtype=torch.int8, device=d),
                    w_scale=torch.empty(N, **f32), static_scale=torch.empty(1, **f32),
                    x_absmax=torch.empty(K, **f32), w_absmax=torch.empty(K, **f32))
    L["xq"] = torch.empty((M, K), dtype=torch.int8, device=d)
    L["xs"] = torch.empty(M, **f32)
    L["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    return L


def _step(layers):
    for L in layers:
        cal = sq.sq_calibrate(L["xc"], L["w"], L["alpha"], out=L["cal"])
        sq.sq_smooth_quantize_act(L["x"], cal["s"], xq=L["xq"], x_scale=L["xs"])
        sq.sq_gemm_w8a8(L["xq"], L["xs"], cal["wq"], cal["w_scale"], y=L["y"])


def _outputs(layers):
    out = []
    for L in layers:
        out += [L["cal"][k].clone() for k in ("s", "wq", "w_scale", "static_scale")]
        out += [L["xq"].clone(), L["xs"].clone(), L["y"].clone()]
    return out


def _clear(layers):
    for L in layers:
        for k in ("s", "wq", "w_scale", "static_scale"):
            L["cal"][k].zero_()
        L["xq"].zero_()
        L["xs"].zero_()
        L["y"].zero_()


def test_graph_replays_match_eager():
    d = dev()
    # a ping-pong, a short-K and a skinny GEMM in one step
    layers = [_layer(d, 300, 512, 1024, 1), _layer(d, 257, 300, 128, 2), _layer(d, 40, 256, 512, 3)]
    _step(layers)
    torch.cuda.synchronize()
    ref = _outputs(layers)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(layers)
    torch.cuda.synchronize()
    other = _layer(d, 130, 192, 256, 4)
    for r in range(4):
        _clear(layers)
        torch.cuda.synchronize()
        say(f"[case] graph replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layers)
        for i, (g, e) in enumerate(zip(got, ref)):
            assert torch.equal(g, e), f"replay {r}: output {i} differs from the eager step"
        _step([other])               # eager library work between the replays
        torch.cuda.synchronize()


def _step_two_streams(layers, side):
    """Calibrations on `side` in order, each linear's quantizer and GEMM on the
    current stream after an event of its own calibration (fork at the start,
    join at the end) -- the overlapped step of the benchmark."""
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    done, cals = [], []
    with torch.cuda.stream(side):
        for L in layers:
            cals.append(sq.sq_calibrate(L["xc"], L["w"], L["alpha"], out=L["cal"]))
            e = torch.cuda.Event()
            e.record(side)
            done.append(e)
    for L, cal, e in zip(layers, cals, done):
        main.wait_event(e)
        sq.sq_smooth_quantize_act(L["x"], cal["s"], xq=L["xq"], x_scale=L["xs"])
        sq.sq_gemm_w8a8(L["xq"], L["xs"], cal["wq"], cal["w_scale"], y=L["y"])
    main.wait_stream(side)


def test_graph_two_streams_replays_match_eager():
    d = dev()
    # GEMMs large enough to keep every CU busy while the later calibrations run
    layers = [_layer(d, 2048, 4096, 2048, 11), _layer(d, 2048, 2048, 4096, 12),
              _layer(d, 1024, 3072, 1024, 13), _layer(d, 300, 512, 1024, 14)]
    _step(layers)
    torch.cuda.synchronize()
    ref = _outputs(layers)
    side = torch.cuda.Stream(d)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step_two_streams(layers, side)
    torch.cuda.synchronize()
    other = _layer(d, 130, 192, 256, 4)
    for r in range(4):
        _clear(layers)
        torch.cuda.synchronize()
        say(f"[case] two-stream graph replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layers)
        for i, (g, e) in enumerate(zip(got, ref)):
            assert torch.equal(g, e), f"replay {r}: output {i} differs from the eager step"
        _step([other])
        torch.cuda.synchronize()
