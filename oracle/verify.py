"""Rejection-sampling verification of a drafted block (oracle; test-only).

The pages: the DFlash drafter proposes a whole block of tokens in one pass
and the backbone verifies the block in one step; the rejection-sampling
verification keeps the output lossless, and the block is capped at 8
("MiMo-V2.5-Pro-FP4-DFlash" model card, §3 "Block-Diffusion Speculative
Decoding (DFlash)").  The pages do not spell the rule out; the reading used
here is the standard speculative-sampling acceptance rule, written from the
losslessness requirement it exists to meet:

  * p_i = softmax of the backbone's logits at block position i (temperature
    1), q_i = the drafter's probabilities there, d_i the drafted token;
  * position i is accepted when u_i * q_i(d_i) < p_i(d_i), i.e. with
    probability min(1, p_i(d_i) / q_i(d_i)), for a uniform u_i in [0, 1);
  * n = the number of leading accepted positions (0..L);
  * the next token is drawn from r(v) = max(0, p_n(v) - q_n(v)) when n < L
    (from p_n itself in the degenerate case where r is all zero), and from
    p_L (the backbone's distribution after the block) when n = L;
  * a draw from weights w uses one uniform u: the smallest token v whose
    running sum of w exceeds u * sum(w) (inverse CDF in vocabulary order);
  * a drafted token outside the vocabulary is rejected.

Every probability is computed in float64.  Random numbers are inputs.
"""

import numpy as np


def softmax64(logits):
    """float64 probabilities of one row of logits (max subtracted)."""
    l = np.asarray(logits, dtype=np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def draw(weights, u):
    """Index drawn from non-negative weights with one uniform u in [0, 1)."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(v, len(w) - 1)


def verify_block(target_logits, draft_probs, draft_tokens, u):
    """One sequence.  target_logits [L+1, V], draft_probs [L, V],
    draft_tokens [L], u [L+1] -> (n accepted, next token)."""
    L = len(draft_tokens)
    n = L
    for i in range(L):
        p = softmax64(target_logits[i])
        d = int(draft_tokens[i])
        if not 0 <= d < len(p):             # a token outside the vocabulary is rejected
            n = i
            break
        if not (float(u[i]) * float(draft_probs[i][d]) < p[d]):
            n = i
            break
    if n < L:
        p = softmax64(target_logits[n])
        w = np.maximum(p - np.asarray(draft_probs[n], dtype=np.float64), 0.0)
        if not w.sum() > 0.0:
            w = p
    else:
        w = softmax64(target_logits[L])
    return n, draw(w, float(u[L]))


def verify_accept(target_logits, draft_probs, draft_tokens, uniforms):
    """Batched: target_logits f32[B, L+1, V], draft_probs f32[B, L, V],
    draft_tokens i32[B, L], uniforms f32[B, L+1] ->
    (accept_len i32[B], next_token i32[B])."""
    B = len(draft_tokens)
    n = np.zeros(B, np.int32)
    t = np.zeros(B, np.int32)
    for b in range(B):
        n[b], t[b] = verify_block(target_logits[b], draft_probs[b], draft_tokens[b], uniforms[b])
    return n, t
