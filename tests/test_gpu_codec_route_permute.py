"""GPU parity of pack/unpack, routing and permutation against the oracle:
bit-exact bytes, ids and lists; routing weights within 2^-20."""

import math

import numpy as np
import pytest
import torch

import workloads
from _gpu import DEV, W_ATOL, dev_bf16, host_bits, say
from oracle import mx as omx
from oracle import permute as operm
from oracle import route as oroute

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import mxfp4_moe_expert_route_amd as m
    m._lib.lib()
    return m


# ---------------------------------------------------------------------------
# unpack


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpack_every_code_scale_pair(mm, dtype):
    say("unpack exhaustive", dtype)
    elem = np.tile(np.arange(16, dtype=np.uint8), 2)
    codes = np.tile(omx.join_nibbles(elem[None, :]), (256, 3))          # K = 96
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 3, axis=1)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = mm.mxfp4_unpack(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), tdt)
    torch.cuda.synchronize()
    want = omx.unpack_to(codes, scales, dtype)
    if dtype == "f32":
        got = y.cpu().numpy().view(np.uint32)
        want = want.view(np.uint32)
        nan_w = np.isnan(want.view(np.float32))
        nan_g = np.isnan(got.view(np.float32))
    else:
        got = host_bits(y)
        nan_w = (want & 0x7FFF) > 0x7F80
        nan_g = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_w, nan_g)
    assert np.array_equal(got[~nan_w], want[~nan_w])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpack_random_matrix(mm, dtype):
    rng = np.random.default_rng(5)
    rows, K = 777, 2080
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 255, (rows, K // 32), dtype=np.uint8)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = mm.mxfp4_unpack(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), tdt)
    want = omx.unpack_to(codes, scales, dtype)
    got = y.cpu().numpy().view(np.uint32) if dtype == "f32" else host_bits(y)
    assert np.array_equal(got, want.view(np.uint32) if dtype == "f32" else want)


# ---------------------------------------------------------------------------
# pack


def pack_inputs(seed, rows=512):
    rng = np.random.default_rng(seed)
    blocks = []
    for i in range(rows * 4):
        kind = i % 8
        if kind == 0:
            b = rng.standard_normal(32) * 2.0 ** rng.integers(-60, 60)
        elif kind == 1:
            b = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.5], 32) * \
                rng.choice([-1, 1], 32) * 2.0 ** rng.integers(-8, 8)
        elif kind == 2:
            b = rng.standard_normal(32) * 2.0 ** rng.integers(-149, -120)
        elif kind == 3:
            b = rng.standard_normal(32) * 2.0 ** rng.integers(100, 127)
        elif kind == 4:
            b = np.where(rng.random(32) < 0.5, -0.0, 0.0)
            b[rng.integers(32)] = rng.standard_normal() * 1e-3
        elif kind == 5:
            b = rng.standard_normal(32)
            b[rng.integers(32)] = rng.choice([np.nan, np.inf, -np.inf])
        elif kind == 6:
            b = np.zeros(32)
        else:
            b = np.round(rng.standard_normal(32) * 64) / 16
        blocks.append(b)
    return np.array(blocks, dtype=np.float64).reshape(rows, 128)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pack_bitexact(mm, dtype):
    v = pack_inputs(1).astype(np.float32)
    if dtype == "f32":
        x = torch.from_numpy(v).to(DEV)
        ref_in = v.astype(np.float64)
    else:
        bits = omx.to_bf16_bits(v.astype(np.float64))
        x = dev_bf16(bits)
        ref_in = omx.bf16_bits_to_f64(bits)
    say("pack", dtype, tuple(v.shape))
    codes, scales = mm.mxfp4_pack(x)
    torch.cuda.synchronize()
    wc, ws = omx.pack(ref_in)
    assert np.array_equal(scales.cpu().numpy(), ws)
    assert np.array_equal(codes.cpu().numpy(), wc)


def test_pack_unpack_roundtrip_on_device(mm):
    rng = np.random.default_rng(3)
    codes = torch.from_numpy(rng.integers(0, 256, (300, 512), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy(rng.integers(110, 140, (300, 32), dtype=np.uint8)).to(DEV)
    y = mm.mxfp4_unpack(codes, scales, torch.float32)
    c2, s2 = mm.mxfp4_pack(y)
    y2 = mm.mxfp4_unpack(c2, s2, torch.float32)
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# routing


def check_route(mm, logits, k):
    ids, w = mm.moe_route_topk(torch.from_numpy(logits).to(DEV), k)
    torch.cuda.synchronize()
    ri, rw = oroute.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ri)
    wg = w.cpu().numpy()
    fin = np.isfinite(rw)
    assert np.array_equal(np.isfinite(wg), fin)
    assert np.abs(wg[fin].astype(np.float64) - rw[fin]).max(initial=0) <= W_ATOL


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_route_on_workload_logits(mm, name):
    cfg = workloads.CONFIGS[name]
    say("route", name)
    x = workloads.gen_x_bits(cfg, 0)
    check_route(mm, workloads.gen_logits(cfg, x, 0), cfg.k)


@pytest.mark.parametrize("E,k", [(1, 1), (2, 2), (64, 1), (65, 65 // 3), (384, 8), (384, 32),
                                 (1000, 7), (1024, 32)])
def test_route_ties_and_special_values(mm, E, k):
    rng = np.random.default_rng(E * 31 + k)
    pool = np.array([0.0, -0.0, 1.5, -2.0, 3.25, 0.5, -math.inf, math.nan], np.float32)
    l = rng.choice(pool, size=(50, E)).astype(np.float32)
    l[:, 0] = 0.125
    l[:5] = rng.standard_normal((5, E)).astype(np.float32)            # some rows without ties
    l[5] = 0.0                                                          # all equal
    check_route(mm, l, k)


# ---------------------------------------------------------------------------
# permutation


def check_permute(mm, ids, E):
    T, k = ids.shape
    got = mm.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    torch.cuda.synchronize()
    ref = operm.permute(ids, E)
    for name, g in zip(("counts", "offsets", "sorted_pairs", "pair_to_row"), got):
        assert np.array_equal(g.cpu().numpy(), ref[name]), name


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_permute_on_workload_routing(mm, name):
    cfg = workloads.CONFIGS[name]
    say("permute", name)
    x = workloads.gen_x_bits(cfg, 0)
    ids, _ = oroute.route_topk(workloads.gen_logits(cfg, x, 0), cfg.k)
    check_permute(mm, ids, cfg.E)


@pytest.mark.parametrize("T,E,k,mode", [(1, 1, 1, "rand"), (3, 5, 5, "rand"), (1000, 1024, 32, "rand"),
                                        (4097, 384, 8, "hot"), (513, 384, 8, "rand"),
                                        (20000, 64, 4, "hot")])
def test_permute_edge_shapes(mm, T, E, k, mode):
    rng = np.random.default_rng(T + E + k)
    if mode == "hot":     # one expert in every token's choice, the rest random
        ids = np.stack([np.concatenate([[0], 1 + rng.permutation(E - 1)[:k - 1]]) for _ in range(T)])
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    check_permute(mm, ids, E)


@pytest.mark.parametrize("T,E,k", [(60, 384, 8), (4000, 384, 8), (1200, 1024, 32)])
def test_permute_drops_out_of_range_ids(mm, T, E, k):
    """Ids outside [0, E) are dropped (one workgroup up to 8192 pairs, ranges
    above): the kept pairs' lists as the oracle's drop mode gives them."""
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    bad = rng.random(ids.shape) < 0.05
    ids = np.where(bad, rng.choice([-1, E, E + 3, -7], size=ids.shape), ids).astype(np.int32)
    got = mm.moe_permute(torch.from_numpy(ids).to(DEV), E)
    torch.cuda.synchronize()
    ref = operm.permute(ids, E, drop_invalid=True)
    kept = int(ref["offsets"][E])
    for name, g in zip(("counts", "offsets", "pair_to_row"), (got[0], got[1], got[3])):
        assert np.array_equal(g.cpu().numpy(), ref[name]), name
    assert np.array_equal(got[2].cpu().numpy()[:kept], ref["sorted_pairs"][:kept])


# ---------------------------------------------------------------------------
# routing and grouping in one call (one fused workgroup up to 16 tokens)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1, 64, 8), (8, 384, 8), (9, 65, 21), (16, 960, 32),
                                   (16, 384, 8), (17, 384, 8), (64, 1024, 32)])
def test_route_permute_matches_oracle_and_two_calls(mm, T, E, k):
    rng = np.random.default_rng(T * 7 + E * 31 + k)
    pool = np.array([0.0, -0.0, 1.5, -2.0, 3.25, 0.5, -math.inf, math.nan], np.float32)
    l = rng.choice(pool, size=(T, E)).astype(np.float32)
    l[: (T + 1) // 2] = rng.standard_normal(((T + 1) // 2, E)).astype(np.float32)
    ld = torch.from_numpy(l).to(DEV)
    got = mm.moe_route_permute(ld, k)
    ids2, w2 = mm.moe_route_topk(ld, k)
    lists2 = mm.moe_permute(ids2, E)
    torch.cuda.synchronize()
    ri, rw = oroute.route_topk(l, k)
    ref = operm.permute(ri, E)
    assert np.array_equal(got[0].cpu().numpy(), ri)
    wg = got[1].cpu().numpy()
    fin = np.isfinite(rw)
    assert np.array_equal(np.isfinite(wg), fin)
    assert np.abs(wg[fin].astype(np.float64) - rw[fin]).max(initial=0) <= W_ATOL
    for name, g in zip(("counts", "offsets", "sorted_pairs", "pair_to_row"), got[2:]):
        assert np.array_equal(g.cpu().numpy(), ref[name]), name
    # bit-identical to the two separate calls, weights included
    assert torch.equal(got[0], ids2)
    assert torch.equal(got[1].view(torch.int32), w2.view(torch.int32))
    for g, g2 in zip(got[2:], lists2):
        assert torch.equal(g, g2)
