"""GPU parity of the batched int8 products of attention (sq_bmm_w8a8;
[Review] §5.6, Fig. 6: the batched matrix multiplications of attention run in
INT8 like the linear layers) against the oracle, bit for bit: small batches
reaching every GEMM kernel (short K for head dimensions 64, 128 and 256,
ping-pong, both ping-pong tiles in one launch, skinny, register-staged), every step granularity and shared (stride 0) operands; and the
OPT-6.7B-shaped attention (32 heads, 2048 tokens, head dimension 128): scores
S = Q K^T and output O = P V with operands quantized per token by
sq_smooth_quantize_act (s = 1), checked on sampled heads.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import w8a8_int8_gemm_colwise_amd as sq
from sqcase import assert_same, dev, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _quant_rows(t3, d):
    """Per-row (per token, or per channel for V^T) int8 codes of a [B, R, C]
    tensor through the library, and the oracle's codes for the same input."""
    B, R, C = t3.shape
    ones = np.ones(C, np.float32)
    xq, xs = sq.sq_smooth_quantize_act(to_dev(t3.reshape(B * R, C), d), to_dev(ones, d))
    return xq.view(B, R, C), xs.view(B, R)


def _oracle_rows(t3):
    B, R, C = t3.shape
    ones = np.ones(C, np.float32)
    q, s, _ = oracle.smooth_quantize_act(t3.reshape(B * R, C), s=ones)
    return q.reshape(B, R, C), s.reshape(B, R)


CASES = [
    # B, M, N, K, x mode, w mode, shared w
    (3, 257, 300, 128, "per_token", "per_channel", False),   # short K (head dim 128)
    (2, 300, 96, 256, "per_token", "per_channel", True),     # short K 256, shared operand
    (2, 200, 300, 384, "per_token", "per_channel", False),   # ping-pong
    (4, 40, 513, 128, "per_token", "per_tensor", False),     # skinny
    (3, 130, 70, 64, "per_token", "per_channel", False),     # short K (head dim 64)
    (2, 150, 90, 192, "per_token", "per_channel", False),    # register-staged (K % 128 != 0)
    (2, 1, 2048, 128, "per_token", "per_channel", False),    # one query token (decode)
    (2, 96, 128, 512, "dynamic_per_tensor", "per_tensor", False),
    # two tile sizes in one launch (256x256 over the first 16384 columns of both entries,
    # 256x128 over the rest): the tile choice counts the batch entries
    (2, 257, 20000, 384, "per_token", "per_channel", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}_{c[1]}x{c[2]}x{c[3]}_{c[4]}_{c[5]}"
                         + ("_shared" if c[6] else ""))
def test_bmm_every_element(case):
    B, M, N, K, xm, wm, shared = case
    d = dev()
    rng = np.random.default_rng(B * 1000 + M + N + K)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((B, M, K)).astype(np.float32) * 2)
    w = datagen.f32_to_bf16_bits(rng.standard_normal((1 if shared else B, N, K)).astype(np.float32))
    xf, wf = oracle.bf16_to_f32(x), oracle.bf16_to_f32(w)
    ones = np.ones(K, np.float32)
    # oracle codes and steps
    if xm == "per_token":
        xq_o, xs_o = _oracle_rows(xf)
    else:
        xq_o, xs_o = zip(*[oracle.quant_dynamic_per_tensor(oracle.act_smooth(xf[b], ones))
                           for b in range(B)])
        xq_o, xs_o = np.stack(xq_o), np.stack(xs_o)
    if wm == "per_channel":
        wq_o, ws_o = _oracle_rows(wf)
    else:
        wq_o, ws_o = zip(*[oracle.quant_dynamic_per_tensor(oracle.act_smooth(wf[b], ones))
                           for b in range(wf.shape[0])])
        wq_o, ws_o = np.stack(wq_o), np.stack(ws_o)
    # GPU: quantize (per entry) and multiply
    if xm == "per_token":
        xq_t, xs_t = _quant_rows(x, d)
    else:
        parts = [sq.sq_smooth_quantize_act(to_dev(x[b], d), to_dev(ones, d), mode=xm)
                 for b in range(B)]
        xq_t = torch.stack([p[0] for p in parts])
        xs_t = torch.stack([p[1] for p in parts])
    if wm == "per_channel":
        wq_t, ws_t = _quant_rows(w, d)
    else:
        parts = [sq.sq_smooth_quantize_act(to_dev(w[b], d), to_dev(ones, d),
                                           mode="dynamic_per_tensor") for b in range(w.shape[0])]
        wq_t = torch.stack([p[0] for p in parts])
        ws_t = torch.stack([p[1] for p in parts])
    if shared:
        wq_t, ws_t = wq_t[0], ws_t[0]
    say(f"[case] bmm B={B} M={M} N={N} K={K} {xm}/{wm} shared={shared}")
    ys = {k: sq.sq_bmm_w8a8(xq_t, xs_t, wq_t, ws_t, mode=xm, out_dtype=k, w_mode=wm)
          for k in ("f32", "bf16", "i32")}
    torch.cuda.synchronize()
    assert_same("xq", to_np(xq_t), xq_o)
    wq_b = np.broadcast_to(wq_o, (B,) + wq_o.shape[1:])
    ws_b = np.broadcast_to(ws_o, (B,) + ws_o.shape[1:])
    for k, yt in ys.items():
        ref = oracle.bmm_w8a8(xq_o, xs_o, wq_b, ws_b, per_token=xm == "per_token",
                              w_per_tensor=wm == "per_tensor", out=k)
        assert_same(f"y[{k}]", to_np(yt), ref)


HEADS, SEQ, HD = 32, 2048, 128


def test_attention_scores_opt67b():
    """S = Q K^T for 32 heads at 2048 tokens, head dimension 128; heads 0 and 31
    compared in full."""
    d = dev()
    q, k, _ = datagen.attention_qkv(HEADS, SEQ, HD, seed=6700)
    qq, qs = _quant_rows(q, d)
    kq, ks = _quant_rows(k, d)
    say("[case] attention scores 32x2048x2048x128")
    s = sq.sq_bmm_w8a8(qq, qs, kq, ks, out_dtype="bf16")
    torch.cuda.synchronize()
    for h in (0, HEADS - 1):
        qo, qso = _oracle_rows(oracle.bf16_to_f32(q[h:h + 1]))
        ko, kso = _oracle_rows(oracle.bf16_to_f32(k[h:h + 1]))
        assert_same(f"q codes head {h}", to_np(qq[h]), qo[0])
        ref = oracle.gemm_w8a8(qo[0], qso[0], ko[0], kso[0], out="bf16")
        assert_same(f"scores head {h}", to_np(s[h]), ref)


def test_attention_output_opt67b():
    """O = P V for 32 heads: P (softmax-shaped rows) quantized per token, V^T
    ([head_dim, tokens]) per channel; heads 3 and 20 compared in full."""
    d = dev()
    _, _, v = datagen.attention_qkv(HEADS, SEQ, HD, seed=6700)
    p = datagen.attention_probs(HEADS, SEQ, SEQ, seed=6800)
    vt = np.ascontiguousarray(np.swapaxes(v, 1, 2))          # [H, d, S] bf16 bits
    pq, ps = _quant_rows(p, d)
    vq, vs = _quant_rows(vt, d)
    say("[case] attention output 32x2048x128x2048")
    o = sq.sq_bmm_w8a8(pq, ps, vq, vs, out_dtype="bf16")
    torch.cuda.synchronize()
    for h in (3, 20):
        po, pso = _oracle_rows(p[h:h + 1])
        vo, vso = _oracle_rows(oracle.bf16_to_f32(vt[h:h + 1]))
        assert_same(f"p codes head {h}", to_np(pq[h]), po[0])
        ref = oracle.gemm_w8a8(po[0], pso[0], vo[0], vso[0], out="bf16")
        assert_same(f"output head {h}", to_np(o[h]), ref)
