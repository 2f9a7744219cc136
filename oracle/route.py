"""Top-k expert routing (oracle; test-only).

The pages give the routing shape only: 384 experts with 8 active per token
(nxbn.cn article, "架构设计与配置详解"; the "MiMo-V2.5-Pro-FP4-DFlash" model
card's §4 "Model Summary" gives hidden size 6144 and 1.02T total / 42B active
parameters) and call the routing dynamic ("动态路由", same article,
"内存优化技巧").  The scoring rule is not on the pages; the reading used
here, listed in the design doc, is:

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
"""

import numpy as np


def _clean(logits):
    l = np.asarray(logits, dtype=np.float64).copy()
    l[np.isnan(l)] = -np.inf
    return l


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
