"""Top-k expert routing (oracle; test-only).

The pages give the routing shape only: 384 experts with 8 active per token
(nxbn.cn article, "架构设计与配置详解"; the "MiMo-V2.5-Pro-FP4-DFlash" model
card's §4 "Model Summary" gives hidden size 6144 and 1.02T total / 42B active
parameters) and call the routing dynamic ("动态路由", same article,
"内存优化技巧").  The scoring rule is not on the pages; the reading used
here is:

  * the input is fp32 router logits [T, E] (the router projection itself is
    upstream of this layer);
  * experts are ordered by descending logit, the lower index first on equal
    logits; -0.0 equals +0.0; a NaN logit ranks as -inf;
  * the k first experts are taken;
  * the weight of each is its softmax probability over all E experts,
    renormalised over the k chosen (so the k weights sum to 1), computed in
    float64 and rounded once to fp32.

Inputs with a +inf logit, or with every logit -inf/NaN, have no defined
weights and are outside the contract.

`router_logits` is the projection in front of the routing (a further step,
not part of the layer's own inputs): the pages give no router form, and the
reading is a linear map of the bf16 hidden state with fp32 weights (plus an
optional per-expert bias), summed exactly in float64 and rounded once to
fp32.
"""

import numpy as np

from .mx import bf16_bits_to_f64


def _clean(logits):
    l = np.asarray(logits, dtype=np.float64).copy()
    l[np.isnan(l)] = -np.inf
    return l


def router_logits(x_bits, w_router, bias=None):
    """x_bits uint16[T, H] (bf16), w_router float32[E, H], bias float32[E] or
    None -> float32[T, E] = fp32(x . w_e (+ bias_e)).

    Every product of a bf16 and an fp32 value is exact in float64 (8 + 24
    significant bits), so the only rounding before the final one is float64
    summation, far below fp32's."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    w = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    out = x @ w.T
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return out.astype(np.float32)


def router_abs_bound(x_bits, w_router):
    """float64[T, E]: sum_h |x_th w_eh|, the scale of fp32 accumulation error."""
    x = np.abs(bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)))
    w = np.abs(np.asarray(w_router, dtype=np.float32).astype(np.float64))
    return x @ w.T


def expert_order(logits):
    """int64[T, E]: experts of each token from best to worst.

    A stable sort of the negated logits keeps equal logits (including -0.0
    against +0.0, and NaN/-inf among themselves) in ascending index order."""
    l = _clean(np.atleast_2d(logits))
    return np.argsort(-l, axis=1, kind="stable")


def route_topk(logits, k):
    """logits float32[T, E] -> (ids int32[T, k], weights float32[T, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    if logits.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if T == 0:
        return np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    l = _clean(logits)
    ids = expert_order(l)[:, :k]
    # softmax over all experts, max subtracted for range
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)
