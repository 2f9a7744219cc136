"""GPU parity of the persistent fused decode layer (moe_mxfp4_decode_layer).

Every output (ids, weights, the four lists, h, y, out) must equal the
multi-launch moe_mxfp4_layer's bit for bit, the layer must match the oracle,
and the workspace must come back zero-filled (the kernel resets its counters
for the next call; its error word stays zero).  Shapes cover one token (most
workgroups start on down units and wait for their tiles), the largest batch
it takes (16 tokens x top-32 over 1024 experts), the largest H and I, ties
in the logits, and the page-shaped 8-token verify step, called several times
in a row on one workspace."""

import dataclasses

import numpy as np
import pytest
import torch

import workloads
from _gpu import DEV, check_layer, dev_bf16, page_layer_weights, say, upload_weights

pytestmark = pytest.mark.gpu

OUTPUTS = ("topk_ids", "topk_w", "counts", "offsets", "sorted_pairs", "pair_to_row", "h", "y",
           "out")


def _fused(mm, cfg, x, logits, w, ws):
    b = mm.LayerBuffers(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, DEV)
    for name in ("h", "y", "out", "topk_w"):
        getattr(b, name).fill_(float("nan"))
    for name in ("topk_ids", "counts", "offsets", "sorted_pairs", "pair_to_row"):
        getattr(b, name).fill_(-7)
    mm.moe_mxfp4_decode_layer(x, logits, cfg.k, w["w13_codes"], w["w13_scales"], w["w2_codes"],
                              w["w2_scales"], ws, buffers=b)
    torch.cuda.synchronize()
    return b


def _same_as_layer(mm, cfg, x, logits, w, ws):
    got = _fused(mm, cfg, x, logits, w, ws)
    ref = mm.moe_mxfp4_layer(x, logits, cfg.k, w["w13_codes"], w["w13_scales"], w["w2_codes"],
                             w["w2_scales"])
    torch.cuda.synchronize()
    for name in OUTPUTS:
        a = getattr(got, name).view(torch.uint8).cpu().numpy()
        r = getattr(ref, name).view(torch.uint8).cpu().numpy()
        assert np.array_equal(a, r), "%s differs from moe_mxfp4_layer" % name
    wsh = ws.cpu().numpy().view(np.uint32)
    assert wsh[2] == 0, "a bounded wait in the kernel gave up"
    assert not wsh.any(), "workspace not left zero-filled"
    return got


@pytest.fixture(scope="module")
def mm():
    import mxfp4_moe_expert_route_amd as m
    m._lib.lib()
    return m


SMALL = [
    # name, (T, H, I, E, k)
    ("dl_one_tok", (1, 2048, 2048, 8, 4)),
    ("dl_t16", (16, 2048, 4096, 64, 8)),
    ("dl_max_pairs", (16, 2048, 2048, 1024, 32)),
    ("dl_h8192", (3, 8192, 2048, 16, 2)),
    ("dl_i8192", (4, 2048, 8192, 8, 2)),
    ("dl_k1", (7, 4096, 2048, 40, 1)),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
def test_decode_layer_small(mm, name, shape):
    T, H, I, E, k = shape
    cfg = workloads.custom_config(name, 900 + [s[0] for s in SMALL].index(name), T, H, I, E, k)
    say("decode layer", name, cfg)
    d = workloads.layer_inputs(cfg, 0)
    w = upload_weights(d)
    ws = mm.decode_layer_workspace(T, H, I, E, k, DEV)
    x = dev_bf16(d["x_bits"])
    lg = torch.from_numpy(d["logits"]).to(DEV)
    _same_as_layer(mm, cfg, x, lg, w, ws)
    check_layer(cfg, d["x_bits"], d["logits"], d, w)        # the multi-launch path vs the oracle


def test_decode_layer_ties(mm):
    cfg = workloads.custom_config("dl_ties", 950, 12, 2048, 2048, 40, 6)
    d = workloads.layer_inputs(cfg, 0)
    rng = np.random.default_rng(950)
    lg = rng.integers(-3, 4, size=(cfg.T, cfg.E)).astype(np.float32)
    lg[0, 5], lg[0, 6] = -0.0, 0.0
    lg[1, :] = np.nan
    lg[1, 7] = 1.0
    w = upload_weights(d)
    ws = mm.decode_layer_workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, DEV)
    _same_as_layer(mm, cfg, dev_bf16(d["x_bits"]), torch.from_numpy(lg).to(DEV), w, ws)
    check_layer(cfg, d["x_bits"], lg, d, w)


def test_decode_layer_page_shaped_repeated(mm):
    """The 8-token verify step of the page-shaped layer, then a 16-token and a
    1-token batch, then the 8-token step again, all on one workspace: each
    equals moe_mxfp4_layer bit for bit and leaves the workspace zero-filled;
    the first is also checked against the oracle on two tokens."""
    from oracle import layer as olayer
    whost, wdev = page_layer_weights()
    base = workloads.CONFIGS["verify_t8"]
    ws = mm.decode_layer_workspace(16, base.H, base.I, base.E, base.k, DEV)
    for i, T in enumerate((8, 16, 1, 8)):
        cfg = base if T == 8 else workloads.custom_config("verify_t%d_dl" % T, 960 + i, T, base.H,
                                                          base.I, base.E, base.k)
        cfg = dataclasses.replace(cfg, layer_id=base.lid) if T != 8 else cfg
        xb = workloads.gen_x_bits(cfg, 0)
        lg = workloads.gen_logits(cfg, xb, 0)
        say("decode layer page-shaped call %d: T=%d" % (i, T))
        got = _same_as_layer(mm, cfg, dev_bf16(xb), torch.from_numpy(lg).to(DEV), wdev, ws)
        if i == 0:
            ref = olayer.layer_forward(xb, lg, whost["w13_codes"], whost["w13_scales"],
                                       whost["w2_codes"], whost["w2_scales"], cfg.k,
                                       tokens=np.array([0, T - 1]))
            out = got.out.cpu().numpy()[[0, T - 1]].astype(np.float64)
            want = ref["out"].astype(np.float64)
            rel = np.linalg.norm(out - want) / np.linalg.norm(want)
            mx = np.abs(out - want).max() / np.sqrt(np.mean(want ** 2))
            say("  oracle on 2 tokens: rel-L2 %.3g, max|d|/RMS %.3g" % (rel, mx))
            assert rel <= 2e-3 and mx <= 1e-2


def test_decode_layer_two_streams(mm):
    """Two persistent layers in flight at once, on two streams with their own
    workspaces and buffers (an 8-token and a 16-token batch of the page-shaped
    layer, three rounds with no synchronisation between).  The second grid
    finds the CUs held by the first, so its workgroups start as the first's
    end (a kernel trace of this test shows the grids of the two streams
    overlapping for about 250 us): the kernel must not depend on its
    workgroups being resident together.  Every output equals moe_mxfp4_layer's bit for bit, no bounded
    wait gives up, and both workspaces come back zero-filled."""
    whost, wdev = page_layer_weights()
    base = workloads.CONFIGS["verify_t8"]
    c16 = workloads.custom_config("verify_t16_two_streams", 970, 16, base.H, base.I, base.E,
                                  base.k)
    c16 = dataclasses.replace(c16, layer_id=base.lid)
    runs = []
    for cfg in (base, c16):
        xb = workloads.gen_x_bits(cfg, 0)
        lg = workloads.gen_logits(cfg, xb, 0)
        x, logits = dev_bf16(xb), torch.from_numpy(lg).to(DEV)
        ws = mm.decode_layer_workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, DEV)
        b = mm.LayerBuffers(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, DEV)
        runs.append((cfg, x, logits, ws, b, torch.cuda.Stream(device=DEV)))
    torch.cuda.synchronize()
    for rnd in range(3):
        for cfg, x, logits, ws, b, s in runs:
            with torch.cuda.stream(s):
                mm.moe_mxfp4_decode_layer(x, logits, cfg.k, wdev["w13_codes"], wdev["w13_scales"],
                                          wdev["w2_codes"], wdev["w2_scales"], ws, buffers=b)
    torch.cuda.synchronize()
    for cfg, x, logits, ws, b, s in runs:
        say("two streams: T=%d" % cfg.T)
        ref = mm.moe_mxfp4_layer(x, logits, cfg.k, wdev["w13_codes"], wdev["w13_scales"],
                                 wdev["w2_codes"], wdev["w2_scales"])
        torch.cuda.synchronize()
        for name in OUTPUTS:
            a = getattr(b, name).view(torch.uint8).cpu().numpy()
            r = getattr(ref, name).view(torch.uint8).cpu().numpy()
            assert np.array_equal(a, r), "T=%d: %s differs from moe_mxfp4_layer" % (cfg.T, name)
        wsh = ws.cpu().numpy().view(np.uint32)
        assert wsh[2] == 0, "T=%d: a bounded wait in the kernel gave up" % cfg.T
        assert not wsh.any(), "T=%d: workspace not left zero-filled" % cfg.T
