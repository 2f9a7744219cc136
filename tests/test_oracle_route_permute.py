"""Pins of the oracle's routing and permutation against brute force, closed
forms and invariants."""

import math

import numpy as np
import pytest

from oracle import permute as operm
from oracle import route as oroute


def brute_order(row):
    """Experts best-first by Python's sort on (-logit, index); NaN ranks as -inf."""
    key = [(-(-math.inf if math.isnan(v) else v), i) for i, v in enumerate(row)]
    return [i for _, i in sorted(key)]


@pytest.mark.parametrize("seed", range(6))
def test_topk_ids_match_brute_force_with_many_ties(seed):
    rng = np.random.default_rng(seed)
    T, E = 40, int(rng.integers(2, 40))
    k = int(rng.integers(1, E + 1))
    # few distinct values -> many ties; include signed zeros, -inf and NaN
    pool = np.array([0.0, -0.0, 1.5, -2.0, 3.25, -math.inf, math.nan], np.float32)
    logits = rng.choice(pool, size=(T, E)).astype(np.float32)
    logits[:, 0] = 0.5                               # at least one finite logit per row
    ids, w = oroute.route_topk(logits, k)
    for t in range(T):
        assert list(ids[t]) == brute_order(logits[t])[:k]


def test_topk_k1_is_argmax_lowest_index_and_kE_is_full_order():
    l = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    ids, w = oroute.route_topk(l, 1)
    assert ids[:, 0].tolist() == [1, 0] and np.all(w == 1.0)
    ids, _ = oroute.route_topk(l, 4)
    assert ids.tolist() == [[1, 2, 3, 0], [0, 1, 2, 3]]


def test_equal_logits_give_first_k_and_uniform_weights():
    ids, w = oroute.route_topk(np.full((3, 10), 0.7, np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == np.float32(0.25))


def test_signed_zero_ties_and_nan_ranks_last():
    ids, _ = oroute.route_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]
    ids, _ = oroute.route_topk(np.array([[0.0, -0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]
    ids, w = oroute.route_topk(np.array([[math.nan, 1.0, 0.0]], np.float32), 3)
    assert ids.tolist() == [[1, 2, 0]]
    assert w[0, 2] == 0.0


def test_two_expert_weight_is_a_sigmoid_of_the_gap():
    rng = np.random.default_rng(1)
    l = (rng.standard_normal((50, 6)) * 3).astype(np.float32)
    ids, w = oroute.route_topk(l, 2)
    for t in range(50):
        a, b = float(l[t, ids[t, 0]]), float(l[t, ids[t, 1]])
        w0 = 1.0 / (1.0 + math.exp(-(a - b)))           # closed form of the renormalised pair
        assert abs(float(w[t, 0]) - w0) <= 2 ** -24
        assert abs(float(w[t, 1]) - (1 - w0)) <= 2 ** -24


def test_weights_sum_to_one_and_do_not_increase():
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((300, 384)) * 1.6).astype(np.float32)
    ids, w = oroute.route_topk(l, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 8 * 2 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)
    # the chosen logits are the 8 largest
    kth = np.sort(l, axis=1)[:, -8]
    assert np.all(np.take_along_axis(l, ids, 1) >= kth[:, None])


def test_shift_invariance():
    rng = np.random.default_rng(4)
    l = rng.integers(-20, 20, (30, 16)).astype(np.float32)
    i1, w1 = oroute.route_topk(l, 5)
    i2, w2 = oroute.route_topk(l + np.float32(64), 5)
    assert np.array_equal(i1, i2) and np.allclose(w1, w2, rtol=0, atol=2 ** -22)


def test_empty_tokens():
    ids, w = oroute.route_topk(np.zeros((0, 8), np.float32), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)


# ---------------------------------------------------------------------------
# permute


@pytest.mark.parametrize("T,E,k,seed", [(16, 8, 2, 0), (1, 4, 4, 1), (37, 64, 8, 2),
                                        (200, 384, 8, 3), (0, 5, 2, 4), (9, 3, 1, 5)])
def test_permute_matches_stable_argsort_construction(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
    d = operm.permute(ids, E)
    flat = ids.reshape(-1)
    # independent construction: stable sort of the expert ids
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(d["counts"], counts)
    assert np.array_equal(d["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(d["sorted_pairs"], order)
    assert np.array_equal(d["sorted_pairs"][d["pair_to_row"]], np.arange(T * k))
    for e in range(E):
        seg = d["sorted_pairs"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        operm.permute(np.array([[0, 5]]), 4)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_permute_drop_invalid_equals_an_extra_expert_removed(seed):
    """Dropping the pairs with ids outside [0, E) gives what routing them to
    an extra expert E gives, with that last segment cut off; on valid input
    the drop mode changes nothing."""
    rng = np.random.default_rng(seed)
    T, E, k = 300, 48, 6
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    assert all(np.array_equal(operm.permute(ids, E, drop_invalid=True)[n], v)
               for n, v in operm.permute(ids, E).items())
    bad = rng.random(ids.shape) < 0.07
    ids_bad = np.where(bad, rng.choice([-1, E, E + 7, -100], size=ids.shape), ids)
    d = operm.permute(ids_bad, E, drop_invalid=True)
    ref = operm.permute(np.where(bad, E, ids), E + 1)          # the bad pairs as expert E
    kept = ref["offsets"][E]
    assert np.array_equal(d["counts"], ref["counts"][:E])
    assert np.array_equal(d["offsets"], ref["offsets"][:E + 1])
    assert d["offsets"][E] == (~bad).sum()
    assert np.array_equal(d["sorted_pairs"][:kept], ref["sorted_pairs"][:kept])
    assert np.all(d["sorted_pairs"][kept:] == -1)
    flat_bad = bad.reshape(-1)
    assert np.all(d["pair_to_row"][flat_bad] == -1)
    assert np.array_equal(d["pair_to_row"][~flat_bad], ref["pair_to_row"][~flat_bad])


# ---- router projection (the step in front of the routing)

def _bf16_bits(v):
    """float32 values that are exactly bf16 -> their bit patterns."""
    b = np.asarray(v, np.float32).view(np.uint32)
    assert np.all(b & 0xffff == 0)
    return (b >> 16).astype(np.uint16)


def test_router_logits_basis_vectors_pick_weight_columns():
    rng = np.random.default_rng(11)
    E, H = 6, 10
    w = rng.standard_normal((E, H)).astype(np.float32)
    x = np.eye(H, dtype=np.float32)                   # token i = unit vector i (1.0 is bf16)
    l = oroute.router_logits(_bf16_bits(x), w)
    assert l.shape == (H, E) and l.dtype == np.float32
    assert np.array_equal(l, w.T)                     # exactly column i of w for token i
    b = rng.standard_normal(E).astype(np.float32)
    lb = oroute.router_logits(_bf16_bits(x), w, b)
    assert np.array_equal(lb, (w.T.astype(np.float64) + b).astype(np.float32))


def test_router_logits_exact_small_integer_case():
    rng = np.random.default_rng(12)
    T, E, H = 7, 5, 64
    x = rng.integers(-2, 3, size=(T, H)).astype(np.float32)
    wq = rng.integers(-4, 5, size=(E, H))
    w = (wq / 8.0).astype(np.float32)                 # multiples of 1/8: every sum exact
    want = (x.astype(np.int64) @ wq.T.astype(np.int64)) / 8.0
    l = oroute.router_logits(_bf16_bits(x), w)
    assert np.array_equal(l.astype(np.float64), want)


def test_router_logits_brute_force_rational():
    from fractions import Fraction
    rng = np.random.default_rng(13)
    T, E, H = 3, 4, 9
    x = rng.standard_normal((T, H)).astype(np.float32)
    x = (x.view(np.uint32) & 0xffff0000).view(np.float32)     # truncate to bf16 values
    w = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    l = oroute.router_logits(_bf16_bits(x), w, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(w[e, h])) for h in range(H))
            exact += Fraction(float(b[e]))
            got = Fraction(float(l[t, e]))
            ulp = np.spacing(np.float32(abs(float(exact)))).astype(np.float64)
            assert abs(got - exact) <= Fraction(float(ulp)) / 2 * Fraction(1001, 1000)


def test_router_abs_bound_dominates_logits():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    x = (x.view(np.uint32) & 0xffff0000).view(np.float32)
    w = rng.standard_normal((3, 32)).astype(np.float32)
    xb = _bf16_bits(x)
    assert np.all(np.abs(oroute.router_logits(xb, w)) <= oroute.router_abs_bound(xb, w) * (1 + 1e-6))
