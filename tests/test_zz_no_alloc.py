"""GPU check of moe_mxfp4_layer_noalloc (the layer entry point that
allocates nothing: its grouping workspace is the library's fixed device
scratch) against moe_mxfp4_layer with a caller workspace.  Both run the same
kernels, so every output must be identical bit for bit.  Two calls in a row
above 8192 token-expert pairs (so the scratch is used), the second smaller,
then one small call that needs no workspace."""

import numpy as np
import pytest
import torch

import workloads
from _gpu import DEV, dev_bf16, dev_u8, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer():
    cfg = workloads.custom_config("noalloc", 90, 2048, 256, 128, 384, 8)
    w = workloads.all_weights(cfg, 0)
    return cfg, {k: dev_u8(v) for k, v in w.items()}


def _inputs(cfg, T):
    c = cfg.with_tokens(T)
    xb = workloads.gen_x_bits(c, 0)
    return dev_bf16(xb), torch.from_numpy(workloads.gen_logits(c, xb, 0)).to(DEV)


def test_noalloc_layer_matches_layer(layer):
    import mxfp4_moe_expert_route_amd as mm
    cfg, w = layer
    args = (w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"])
    for T in (2048, 1200, 16):
        R = T * cfg.k
        say("noalloc layer: T=%d (R=%d, workspace %d B)"
            % (T, R, mm.moe_permute_workspace_bytes(T, cfg.E, cfg.k)))
        x, logits = _inputs(cfg, T)
        ref = mm.moe_mxfp4_layer(x, logits, cfg.k, *args)
        got = mm.LayerBuffers(T, cfg.H, cfg.I, cfg.E, cfg.k, DEV)
        for name in ("h", "y", "out"):
            getattr(got, name).fill_(float("nan"))
        for name in ("topk_ids", "counts", "offsets", "sorted_pairs", "pair_to_row"):
            getattr(got, name).fill_(-7)
        torch.cuda.synchronize()
        mm.moe_mxfp4_layer_noalloc(x, logits, cfg.k, *args, got)
        torch.cuda.synchronize()
        for name in ("topk_ids", "topk_w", "counts", "offsets", "sorted_pairs", "pair_to_row",
                     "h", "y", "out"):
            a = getattr(got, name).view(torch.uint8).cpu().numpy()
            b = getattr(ref, name).view(torch.uint8).cpu().numpy()
            assert np.array_equal(a, b), "T=%d: %s differs" % (T, name)
        assert int(got.offsets[-1].item()) == R
