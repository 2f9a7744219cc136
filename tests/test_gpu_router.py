"""GPU parity of moe_router_topk (router projection, then top-k routing)
against the oracle.

Logits: within fp32 accumulation error of the exact sum, |err| <= 2^-16 *
sum_h |x_th w_eh| (the kernel's per-lane fma chains are at most H/256 long,
or 32-term chains then one add per 32, at most 224 terms in a chain at H =
6144; 2^-16 is 256 units in the last place of that scale, a dropped term
of the sum is about 2^-12.6 of it).
Routing: ids bit-exact and weights within 2^-20 of the oracle's routing of
the logits the GPU wrote, which is how moe_route_topk is pinned; logits
bitwise equal across two calls."""

import numpy as np
import pytest
import torch

import workloads
from _gpu import DEV, W_ATOL, dev_bf16, say
from oracle import route as oroute

pytestmark = pytest.mark.gpu

CASES = [
    # name, (T, H, E, k) or None for a named workload
    ("tiny_t16", None),
    ("ragged_t13", (13, 100, 7, 3)),       # H not a multiple of 256, E not of 4
    ("blocks32_t70", (70, 520, 33, 4)),    # the 32-token blocks, a ragged last block
    ("narrow_t7", (7, 132, 19, 2)),        # one block, H % 8 == 4: 8-byte loads of x
    ("two_pass_t6", (6, 6152, 11, 2)),     # one block, a second pass over H
    ("wide_e", (5, 64, 1024, 32)),
    ("one_expert", (9, 32, 1, 1)),
    ("verify_t8", None),
    ("verify_t64", None),
    ("zipf_t512", None),                   # with the skewing per-expert bias
    ("prefill_t8192", None),
]


@pytest.fixture(scope="module")
def mm():
    import mxfp4_moe_expert_route_amd as m
    m._lib.lib()
    return m


@pytest.mark.parametrize("name,shape", CASES, ids=[c[0] for c in CASES])
def test_router_topk_matches_oracle(mm, name, shape):
    if shape is None:
        cfg = workloads.CONFIGS[name]
        T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
        x_bits = workloads.gen_x_bits(cfg, 0)
        w = workloads.gen_router(cfg, 0)
        bias = workloads.gen_bias(cfg, 0).astype(np.float32) if cfg.routing != "uniform" else None
    else:
        # shapes the layer does not take (H only a multiple of 4): drawn here
        T, H, E, k = shape
        rng = np.random.default_rng(900 + [c[0] for c in CASES].index(name))
        x_bits = workloads.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        w = rng.normal(0.0, 0.02, size=(E, H)).astype(np.float32)
        bias = rng.normal(0.0, 1.0, size=E).astype(np.float32)
    say("router", name, T, H, E, k)
    xd = dev_bf16(x_bits)
    wd = torch.from_numpy(w).to(DEV)
    bd = torch.from_numpy(bias).to(DEV) if bias is not None else None
    logits, ids, tw = mm.moe_router_topk(xd, wd, k, bd)
    logits2, _, _ = mm.moe_router_topk(xd, wd, k, bd)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), logits2.cpu().numpy().view(np.uint32)), \
        "logits differ between two calls"

    want = oroute.router_logits(x_bits, w, bias)
    bound = oroute.router_abs_bound(x_bits, w)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = 2.0 ** -16 * bound + 1e-30
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    say("  max |err| %.3g, worst err/tol %.3g at %s" % (err.max(), (err / tol).max(), worst))
    assert np.all(err <= tol), "logits outside fp32 accumulation error"

    rid, rw = oroute.route_topk(got, k)
    assert np.array_equal(ids.cpu().numpy(), rid), "ids differ from routing the written logits"
    assert np.max(np.abs(tw.cpu().numpy() - rw)) <= W_ATOL
