"""Pins of the block verification oracle: losslessness computed exactly
(the emitted token's distribution equals the backbone's), special cases and a
brute-force sampler."""

import numpy as np
import pytest

from oracle import verify as ov


def _probs(rng, V, scale=1.5):
    l = rng.normal(0.0, scale, V)
    e = np.exp(l - l.max())
    return l.astype(np.float32), (e / e.sum())


def _first_token_distribution(target_logits0, q0, n_u=4000):
    """P(first emitted token = v) when d_0 ~ q0: the acceptance uniform and
    the sampling uniform are integrated on midpoint grids."""
    V = len(q0)
    out = np.zeros(V)
    us = (np.arange(n_u) + 0.5) / n_u
    tl = np.stack([target_logits0, target_logits0])         # [L+1 = 2, V]
    for d in range(V):
        if q0[d] == 0:
            continue
        for u0 in us[::40]:                                  # acceptance uniform
            # accepted: emits d; rejected: the residual draw, integrated exactly
            n, _ = ov.verify_block(tl, q0[None, :].astype(np.float32), [d], [u0, 0.5])
            if n == 1:
                out[d] += q0[d] / len(us[::40])
            else:
                p = ov.softmax64(target_logits0)
                w = np.maximum(p - q0.astype(np.float32).astype(np.float64), 0)
                if w.sum() == 0:
                    w = p
                cnt = np.bincount([ov.draw(w, u1) for u1 in us], minlength=V) / len(us)
                out += q0[d] / len(us[::40]) * cnt
    return out


@pytest.mark.parametrize("seed", range(3))
def test_first_token_is_distributed_as_the_backbone(seed):
    rng = np.random.default_rng(seed)
    V = 6
    tl, p = _probs(rng, V)
    _, q = _probs(rng, V, 2.0)
    q = q.astype(np.float32)
    got = _first_token_distribution(tl, q)
    assert np.allclose(got, ov.softmax64(tl), atol=0.02), (got, ov.softmax64(tl))


def test_drafter_equal_to_backbone_accepts_everything():
    rng = np.random.default_rng(5)
    L, V = 8, 50
    tl = rng.normal(0, 2, (L + 1, V)).astype(np.float32)
    q = np.stack([ov.softmax64(tl[i]) for i in range(L)]).astype(np.float32)
    for s in range(20):
        d = [int(rng.integers(V)) for _ in range(L)]
        u = rng.random(L + 1).astype(np.float32) * 0.999
        # q = fp32(p): u*q < p holds except where rounding puts q above p by an ulp and u ~ 1
        n, t = ov.verify_block(tl, q, d, u)
        assert n == L
        assert t == ov.draw(ov.softmax64(tl[L]), float(u[L]))


def test_token_the_backbone_rules_out_is_rejected_and_not_redrawn():
    V = 5
    tl = np.array([[0, 0, -np.inf, 0, 0], [1, 2, 3, 4, 5]], np.float32)
    q = np.array([[0.1, 0.1, 0.6, 0.1, 0.1]], np.float32)
    for u0 in (0.0, 0.5, 0.99):
        for u1 in (0.0, 0.3, 0.99):
            n, t = ov.verify_block(tl, q, [2], [u0, u1])
            assert n == 0 and t != 2


def test_draw_matches_brute_force_walk():
    rng = np.random.default_rng(9)
    for _ in range(200):
        w = rng.random(17) * (rng.random(17) < 0.6)
        if w.sum() == 0:
            continue
        u = rng.random()
        run, pick = 0.0, len(w) - 1
        for v, x in enumerate(w):
            run += x
            if run > u * w.sum():
                pick = v
                break
        assert ov.draw(w, u) == pick


def test_one_hot_backbone_accepts_exactly_its_token():
    V, L = 7, 3
    tl = np.full((L + 1, V), -np.inf, np.float32)
    for i, tok in enumerate([3, 1, 4, 2]):
        tl[i, tok] = 0.0
    q = np.full((L, V), 1.0 / V, np.float32)
    n, t = ov.verify_block(tl, q, [3, 1, 5], [0.9, 0.9, 0.9, 0.4])
    assert n == 2 and t == 4        # position 2 drafted 5, the backbone only allows 4
    n, t = ov.verify_block(tl, q, [3, 1, 4], [0.9, 0.9, 0.9, 0.4])
    assert n == 3 and t == 2        # all accepted, bonus from position 3


def test_token_outside_vocabulary_is_rejected():
    V = 4
    tl = np.zeros((3, V), np.float32)
    q = np.full((2, V), 0.25, np.float32)
    assert ov.verify_block(tl, q, [V, 0], [0.0, 0.0, 0.5])[0] == 0
    assert ov.verify_block(tl, q, [1, -1], [0.0, 0.0, 0.5])[0] == 1
