"""The MXFP4 MoE expert layer by its plain definition (oracle; test-only).

What the pages fix: the experts of each MoE layer are stored in MXFP4 with
block size 32 while activations stay in higher precision ("MiMo-V2.5-Pro-
FP4-DFlash" model card, §1 Introduction and §2 "FP4 Quantization"; the
serving example's --dtype bfloat16 in §5 "Deployment"); 384 experts, 8 active
per token (nxbn.cn article, "架构设计与配置详解"); hidden size 6144 (§4 "Model
Summary").  The backbone verifies a block of 8 drafted tokens per sequence in
one step (§3, mask block capped at 8), so a decode step runs this layer on
8 tokens per sequence.

Readings, where the pages are silent:
  * each expert is a SwiGLU FFN without biases: g = W_gate x, u = W_up x,
    h = silu(g) * u with silu(g) = g / (1 + exp(-g)), y = W_down h;
  * the stacked gate/up matrix W13 [2I, H] holds gate rows 0..I-1 then up
    rows I..2I-1; W2 is [H, I]; MX blocks run along the last axis;
  * x is bf16; h is stored as bf16 (rounded once, RNE) because the down
    projection consumes bf16 activations; y and the layer output are fp32;
  * out_t = sum_j w_tj * y_tj over the token's k chosen experts, with the
    fp32 routing weights;
  * no shared expert, no routed scaling factor.

Computation: products of bf16 inputs and exactly dequantised weights are
exact in float64, so only the summations round; each expert's matrices are
dequantised once and applied to the tokens routed to it with a float64
matrix product.
"""

import numpy as np

from . import mx
from .route import route_topk


def silu(g):
    return g / (1.0 + np.exp(-g))


def gate_up_swiglu(x64, w13_codes, w13_scales):
    """Rows x64 float64[n, H] against 2C weight rows (C gate rows, then the up
    rows of the same C columns) -> h_bits uint16[n, C] = bf16(silu(g) * u)."""
    W13 = mx.unpack(w13_codes, w13_scales)      # [2C, H]
    C = W13.shape[0] // 2
    g = x64 @ W13[:C].T
    u = x64 @ W13[C:].T
    return mx.to_bf16_bits(silu(g) * u)


def expert_ffn(x64, w13_codes, w13_scales, w2_codes, w2_scales):
    """One expert on rows x64 float64[n, H] -> (h_bits uint16[n, I], y float32[n, H])."""
    h_bits = gate_up_swiglu(x64, w13_codes, w13_scales)
    h = mx.bf16_bits_to_f64(h_bits)
    W2 = mx.unpack(w2_codes, w2_scales)         # [H, I]
    y = mx.to_f32(h @ W2.T)
    return h_bits, y


def layer_forward(x_bits, logits, w13_codes, w13_scales, w2_codes, w2_scales, k,
                  tokens=None):
    """Full layer.

    x_bits      uint16[T, H] bf16 activations
    logits      float32[T, E] router logits
    w13_codes   [E, 2I, H/2] uint8 (indexable by expert; may be lazy)
    w13_scales  [E, 2I, H/32] uint8
    w2_codes    [E, H, I/2] uint8
    w2_scales   [E, H, I/32] uint8
    tokens      optional 1-D token indices: the FFN is evaluated only for them
                (routing is still computed for every token)

    Returns dict with ids, w (all tokens) and, for the evaluated tokens in the
    order given, tok, h_bits [n, k, I], y [n, k, H] fp32, out [n, H] fp32.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    logits = np.asarray(logits, dtype=np.float32)
    T, H = x_bits.shape
    ids, w = route_topk(logits, k)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    X = mx.bf16_bits_to_f64(x_bits[tok])
    sel = ids[tok]                                # [n, k]
    y = None
    h_bits = None
    for e in np.unique(sel):
        rows, slots = np.nonzero(sel == e)
        hb, ye = expert_ffn(X[rows], w13_codes[e], w13_scales[e],
                            w2_codes[e], w2_scales[e])
        if y is None:
            y = np.zeros((n, k, ye.shape[1]), np.float32)
            h_bits = np.zeros((n, k, hb.shape[1]), np.uint16)
        y[rows, slots] = ye
        h_bits[rows, slots] = hb
    if y is None:                                 # no tokens evaluated
        I = np.asarray(w2_codes[0]).shape[-1] * 2 if len(w2_codes) else 0
        y = np.zeros((n, k, H), np.float32)
        h_bits = np.zeros((n, k, I), np.uint16)
    out = np.zeros((n, H), np.float64)
    wt = w[tok].astype(np.float64)
    for j in range(k):
        out += wt[:, j:j + 1] * y[:, j].astype(np.float64)
    return {"ids": ids, "w": w, "tok": tok, "h_bits": h_bits, "y": y,
            "out": mx.to_f32(out)}
