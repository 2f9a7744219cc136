"""GPU parity of dflash_verify_accept against the oracle.

The GPU decides in fp32 and the oracle in float64, so a decision may differ
only where the exact margin is within fp32 rounding: accept lengths must
match wherever every tested position's margin |p - u q| exceeds 1e-5 of
max(p, u q); the drawn token must match wherever the draw target u * sum(w)
lies more than 1e-5 * sum(w) from the token's cumulative-sum boundaries, and
otherwise must be a token whose float64 interval reaches the target within
that tolerance.  Results are bitwise repeatable."""

import numpy as np
import pytest
import torch

import workloads
from _gpu import DEV, say
from oracle import verify as ov

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, L, V, logit_std, draft_noise
    ("small_vocab", 6, 8, 64, 1.0, 0.3),
    ("ragged_parts", 5, 8, 1000, 2.0, 0.3),    # 250 chunks: parts of 8, the last short
    ("one_position", 5, 1, 96, 2.0, 0.5),
    ("wide_block", 3, 32, 256, 2.0, 0.2),
    ("near_equal_draft", 4, 8, 512, 3.0, 0.01),
    ("verify_t8", 1, 8, workloads.VERIFY_VOCAB, 3.0, 0.35),
    ("verify_t64", 8, 8, workloads.VERIFY_VOCAB, 3.0, 0.35),
    ("poor_draft", 8, 8, workloads.VERIFY_VOCAB, 3.0, 1.5),
]


@pytest.fixture(scope="module")
def mm():
    import mxfp4_moe_expert_route_amd as m
    m._lib.lib()
    return m


def _check(target, draft, tokens, uniforms, n_gpu, t_gpu):
    B, L1, V = target.shape
    L = L1 - 1
    exact = 0
    for b in range(B):
        n_or, t_or = ov.verify_block(target[b], draft[b], tokens[b], uniforms[b])
        # margins of the positions the oracle tested
        close = False
        for i in range(min(n_or + 1, L)):
            p = ov.softmax64(target[b, i])
            d = int(tokens[b, i])
            pd = p[d] if 0 <= d < V else 0.0
            uq = float(uniforms[b, i]) * float(draft[b, i, d]) if 0 <= d < V else 0.0
            if abs(pd - uq) <= 1e-5 * max(pd, uq):
                close = True
        if not close:
            assert n_gpu[b] == n_or, (b, n_gpu[b], n_or)
        n = int(n_gpu[b])
        p = ov.softmax64(target[b, n])
        w = np.maximum(p - draft[b, n].astype(np.float64), 0.0) if n < L else p
        if n < L and not w.sum() > 0:
            w = p
        c = np.cumsum(w)
        tgt = float(uniforms[b, L]) * c[-1]
        tol = 1e-5 * c[-1]
        v = int(t_gpu[b])
        lo = c[v - 1] if v > 0 else 0.0
        if n == n_or and abs(lo - tgt) > tol and abs(c[v] - tgt) > tol and \
                abs((c[t_or - 1] if t_or > 0 else 0.0) - tgt) > tol and abs(c[t_or] - tgt) > tol:
            assert v == t_or, (b, v, t_or)
            exact += 1
        else:
            assert lo - tol <= tgt <= c[v] + tol, (b, v, lo, c[v], tgt)
            assert w[v] >= -tol
    return exact


@pytest.mark.parametrize("name,B,L,V,std,noise", CASES, ids=[c[0] for c in CASES])
def test_verify_matches_oracle(mm, name, B, L, V, std, noise):
    say("verify", name, B, L, V)
    target, draft, tokens, uniforms = workloads.gen_verify_inputs(B, L, V, 0, std, noise)
    if name == "small_vocab":
        tokens[0, 3] = V + 5                       # out of range: rejected
        tokens[1, 0] = -1
    td = torch.from_numpy(target).to(DEV)
    dd = torch.from_numpy(draft).to(DEV)
    kd = torch.from_numpy(tokens).to(DEV)
    ud = torch.from_numpy(uniforms).to(DEV)
    n1, t1 = mm.dflash_verify_accept(td, dd, kd, ud)
    n2, t2 = mm.dflash_verify_accept(td, dd, kd, ud)
    torch.cuda.synchronize()
    n1, t1 = n1.cpu().numpy(), t1.cpu().numpy()
    assert np.array_equal(n1, n2.cpu().numpy()) and np.array_equal(t1, t2.cpu().numpy())
    exact = _check(target, draft, tokens, uniforms, n1, t1)
    say("  accept lengths", n1.tolist(), "tokens compared exactly:", exact, "of", B)
    if name == "small_vocab":
        assert n1[0] <= 3 and n1[1] == 0
