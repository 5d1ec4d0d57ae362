"""Seeded synthetic inputs for the SmoothQuant W8A8 linear-layer path.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic.  Both the CPU oracle and the GPU path consume exactly
the arrays produced here (fp32 arrays, or bf16 bit patterns as uint16).

Distributions follow the pages' description of LLM activations: most channels
small ([Edge] §一.1: 99% of channels within [-2, 2]), a fixed set of 0.1%-0.5%
of channels reaching +-50..+-120 ([Edge] §一.1; [Review] §4 observation 3 and
Fig. 4: outliers persist in fixed channels), and weights that are flat and
easy to quantize ([Review] §4 observation 1).  The pages measure on real
models and datasets (OPT, Llama, the Pile); these seeded tensors stand in for
them.

Recipe (shared by every configuration):
  * seeds: base S = 1000*c for configuration c (1..5), plus 10*l for the l-th
    linear of a configuration; calibration X uses S, evaluation X uses S+1,
    W uses S+2, gamma/beta S+3, the outlier channel set S+5;
  * outlier channel count max(1, round(f*K)); outlier entries REPLACE the base
    entries in those channels; magnitudes U(50, 120); the sign is either fixed
    per channel (drawn once with the channel set) or random per entry;
  * bf16 tensors are drawn in fp32 and rounded to bf16 (nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

OUTLIER_LO, OUTLIER_HI = 50.0, 120.0


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer of a synthetic workload."""
    name: str
    K: int                      # input channels
    N: int                      # output channels
    M: int                      # evaluation tokens
    T: int                      # calibration tokens
    x_std: float                # base activation std
    x_clip: float | None        # clip base activations to [-c, c] (None: no clip)
    x_dtype: str                # "f32" | "bf16"
    w_std: float
    w_dtype: str
    outlier_frac: float | None  # fraction of channels, or None when n_outliers given
    n_outliers_fixed: int | None
    outlier_sign: str           # "channel" (fixed per channel) | "entry" (random per entry)
    alpha: float
    mode: str                   # "static" | "per_token"
    ln: bool = False            # LayerNorm-mode activation side
    seed_base: int = 0

    @property
    def n_outliers(self) -> int:
        if self.n_outliers_fixed is not None:
            return self.n_outliers_fixed
        return max(1, int(round(self.outlier_frac * self.K)))


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    layers: tuple
    notes: str = ""
    extra: dict = field(default_factory=dict)


def _base(c: int, l: int) -> int:
    return 1000 * c + 10 * l


def _single_linear_512() -> Workload:
    spec = LayerSpec("linear_512", K=512, N=512, M=16, T=64, x_std=0.5, x_clip=None,
                     x_dtype="f32", w_std=0.02, w_dtype="f32", outlier_frac=None,
                     n_outliers_fixed=2, outlier_sign="channel", alpha=0.5, mode="static",
                     seed_base=_base(1, 0))
    return Workload(1, "single_linear_512", (spec,),
                    "fp32 64x512 calibration, 16x512 evaluation, 512x512 W, static scale")


def _opt67b_prefill() -> Workload:
    shapes = (("qkv", 4096, 12288), ("out_proj", 4096, 4096), ("fc1", 4096, 16384),
              ("fc2", 16384, 4096))
    layers = tuple(
        LayerSpec(n, K=k, N=nn, M=2048, T=512, x_std=1.0, x_clip=2.0, x_dtype="bf16",
                  w_std=0.02, w_dtype="bf16", outlier_frac=0.001, n_outliers_fixed=None,
                  outlier_sign="entry", alpha=0.5, mode="per_token", seed_base=_base(2, l))
        for l, (n, k, nn) in enumerate(shapes))
    return Workload(2, "opt6.7b_prefill_m2048", layers,
                    "OPT-6.7B-shaped prefill linears, 2048 tokens, per-token dynamic")


def _decode_70b_ffn(M: int = 64) -> Workload:
    shapes = (("ffn_up", 8192, 28672), ("ffn_down", 28672, 8192))
    layers = tuple(
        LayerSpec(n, K=k, N=nn, M=M, T=512, x_std=0.5, x_clip=None, x_dtype="bf16",
                  w_std=0.02, w_dtype="bf16", outlier_frac=0.003, n_outliers_fixed=None,
                  outlier_sign="channel", alpha=0.5, mode="per_token", seed_base=_base(3, l))
        for l, (n, k, nn) in enumerate(shapes))
    return Workload(3, f"70b_ffn_decode_m{M}", layers,
                    "decode-shaped W8A8, M in {1,8,32,64}", extra={"M_values": (1, 8, 32, 64)})


def _opt175b_layer() -> Workload:
    shapes = (("qkv", 12288, 36864), ("out_proj", 12288, 12288), ("fc1", 12288, 49152),
              ("fc2", 49152, 12288))
    layers = tuple(
        LayerSpec(n, K=k, N=nn, M=4096, T=512, x_std=1.0, x_clip=2.0, x_dtype="bf16",
                  w_std=0.015, w_dtype="bf16", outlier_frac=0.002, n_outliers_fixed=None,
                  outlier_sign="entry", alpha=0.5, mode="per_token", seed_base=_base(4, l))
        for l, (n, k, nn) in enumerate(shapes))
    return Workload(4, "opt175b_layer_m4096", layers,
                    "OPT-175B-shaped full layer, 4096 tokens, one GPU, no sharding")


ALPHA_SWEEP = (0.0, 0.25, 0.5, 0.75, 0.85, 1.0)


def _ln_pipeline_8192(alpha: float = 0.5, T: int = 65536) -> Workload:
    spec = LayerSpec("ln_linear_8192", K=8192, N=22016, M=4096, T=T, x_std=1.0, x_clip=2.0,
                     x_dtype="bf16", w_std=0.02, w_dtype="bf16", outlier_frac=0.005,
                     n_outliers_fixed=None, outlier_sign="entry", alpha=alpha,
                     mode="per_token", ln=True, seed_base=_base(5, 0))
    return Workload(5, "ln_pipeline_h8192", (spec,),
                    "LayerNorm-fused smoothing at hidden 8192, alpha sweep",
                    extra={"alphas": ALPHA_SWEEP})


def workload(cid: int, **kw) -> Workload:
    return {1: _single_linear_512, 2: _opt67b_prefill, 3: _decode_70b_ffn,
            4: _opt175b_layer, 5: _ln_pipeline_8192}[cid](**kw)


# ---- drawing ----------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def outlier_set(spec: LayerSpec):
    """(channel indices, per-channel signs) shared by calibration and evaluation."""
    g = _rng(spec.seed_base + 5)
    ch = np.sort(g.choice(spec.K, size=spec.n_outliers, replace=False))
    sign = g.choice(np.array([-1.0, 1.0], np.float32), size=spec.n_outliers)
    return ch, sign


def _activations_f32(spec: LayerSpec, rows: int, seed: int, chunk: int = 8192) -> np.ndarray:
    """Base N(0, std^2) (optionally clipped) with the outlier channels replaced."""
    out = np.empty((rows, spec.K), np.float32)
    r0 = 0
    for blk in _activations_iter(spec, rows, seed, chunk):
        out[r0:r0 + blk.shape[0]] = blk
        r0 += blk.shape[0]
    return out


def ln_params(spec: LayerSpec):
    """gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1^2), fp32 [K]."""
    g = _rng(spec.seed_base + 3)
    gamma = g.uniform(0.5, 1.5, size=spec.K).astype(np.float32)
    beta = (g.standard_normal(spec.K) * 0.1).astype(np.float32)
    return gamma, beta


def bias(spec: LayerSpec) -> np.ndarray:
    """Output bias of the linear, N(0, 0.1^2) fp32 [N] (seed base + 4)."""
    return (_rng(spec.seed_base + 4).standard_normal(spec.N) * 0.1).astype(np.float32)


def _model_layernorm_f32(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                         eps: float = 1e-5) -> np.ndarray:
    """The model's own (unsmoothed) LayerNorm in fp32 numpy.  Used only to
    synthesise calibration activations as a calibration run would record them
    at the input of the linear; it is not a step of the smoothed path (which
    folds 1/s into gamma and beta and fixes its own reduction order)."""
    mu = x.mean(axis=1, keepdims=True, dtype=np.float32)
    d = x - mu
    var = (d * d).mean(axis=1, keepdims=True, dtype=np.float32)
    return d / np.sqrt(var + np.float32(eps)) * gamma[None, :] + beta[None, :]


def calibration_x(spec: LayerSpec, T: int | None = None) -> np.ndarray:
    """Calibration activations [T, K] in the layer's input dtype."""
    T = spec.T if T is None else T
    if not spec.ln:
        return _cast(_activations_f32(spec, T, spec.seed_base), spec.x_dtype)
    gamma, beta = ln_params(spec)
    out = np.empty((T, spec.K), np.uint16 if spec.x_dtype == "bf16" else np.float32)
    chunk = 4096
    g_seed = spec.seed_base
    pre = _activations_iter(spec, T, g_seed, chunk)
    r0 = 0
    for blk in pre:
        out[r0:r0 + blk.shape[0]] = _cast(_model_layernorm_f32(blk, gamma, beta), spec.x_dtype)
        r0 += blk.shape[0]
    return out


def _activations_iter(spec: LayerSpec, rows: int, seed: int, chunk: int):
    g = _rng(seed)
    ch, sign = outlier_set(spec)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        blk = g.standard_normal((r1 - r0, spec.K), dtype=np.float32)
        blk *= np.float32(spec.x_std)
        if spec.x_clip is not None:
            np.clip(blk, -spec.x_clip, spec.x_clip, out=blk)
        mag = g.uniform(OUTLIER_LO, OUTLIER_HI, size=(r1 - r0, ch.size)).astype(np.float32)
        if spec.outlier_sign == "channel":
            sgn = sign[None, :]
        else:
            sgn = g.choice(np.array([-1.0, 1.0], np.float32), size=(r1 - r0, ch.size))
        blk[:, ch] = mag * sgn
        yield blk


def eval_x(spec: LayerSpec, M: int | None = None) -> np.ndarray:
    """Runtime activations [M, K] (pre-LayerNorm tokens in LayerNorm mode)."""
    M = spec.M if M is None else M
    return _cast(_activations_f32(spec, M, spec.seed_base + 1), spec.x_dtype)


def weights(spec: LayerSpec) -> np.ndarray:
    """W [N, K] (out x in), N(0, w_std^2), in the layer's weight dtype."""
    g = _rng(spec.seed_base + 2)
    out = np.empty((spec.N, spec.K), np.uint16 if spec.w_dtype == "bf16" else np.float32)
    chunk = max(1, (1 << 24) // spec.K)
    for r0 in range(0, spec.N, chunk):
        r1 = min(spec.N, r0 + chunk)
        blk = g.standard_normal((r1 - r0, spec.K), dtype=np.float32) * np.float32(spec.w_std)
        out[r0:r1] = _cast(blk, spec.w_dtype)
    return out


def random_layer(M: int, N: int, K: int, seed: int, x_dtype: str = "bf16",
                 w_dtype: str = "bf16", n_outliers: int = 2, T: int = 32,
                 alpha: float = 0.5, mode: str = "per_token", ln: bool = False) -> LayerSpec:
    """A small ragged layer for parity tests (sizes not tied to a workload)."""
    return LayerSpec(f"rand_{M}x{N}x{K}_{seed}", K=K, N=N, M=M, T=T, x_std=1.0, x_clip=2.0,
                     x_dtype=x_dtype, w_std=0.02, w_dtype=w_dtype, outlier_frac=None,
                     n_outliers_fixed=min(n_outliers, K), outlier_sign="entry", alpha=alpha,
                     mode=mode, ln=ln, seed_base=seed)


# ---- attention products ([Review] §5.6, Fig. 6) --------------------------------------

def attention_qkv(heads: int, seq: int, head_dim: int, seed: int, n_outliers: int = 2):
    """Q, K, V of one attention layer as bf16 bit patterns [heads, seq, head_dim]:
    N(0, 1) entries, with n_outliers fixed channels of Q and K scaled by
    U(5, 15) (query/key outliers persist per channel); seeds seed, seed+1, seed+2."""
    out = []
    for j, name in enumerate(("q", "k", "v")):
        g = _rng(seed + j)
        t = g.standard_normal((heads, seq, head_dim)).astype(np.float32)
        if name != "v" and n_outliers:
            ch = g.choice(head_dim, size=n_outliers, replace=False)
            t[:, :, ch] *= g.uniform(5.0, 15.0, size=n_outliers).astype(np.float32)
        out.append(f32_to_bf16_bits(t))
    return tuple(out)


def attention_probs(heads: int, seq_q: int, seq_k: int, seed: int) -> np.ndarray:
    """Softmax-shaped attention probabilities [heads, seq_q, seq_k] fp32: each row
    is softmax of N(0, 2^2) logits, computed in fp32 per head (seed + head)."""
    p = np.empty((heads, seq_q, seq_k), np.float32)
    for h in range(heads):
        z = _rng(seed + h).standard_normal((seq_q, seq_k)).astype(np.float32) * np.float32(2.0)
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z, dtype=np.float32)
        p[h] = e / e.sum(axis=1, keepdims=True, dtype=np.float32)
    return p
