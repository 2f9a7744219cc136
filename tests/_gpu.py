"""Helpers shared by the GPU parity tests: device upload, tolerance checks,
and a cache of the page-shaped layer's weights (generated once per session)."""

import sys

import numpy as np
import torch

import workloads
from oracle import layer as olayer
from oracle import mx as omx
from oracle import permute as operm

DEV = torch.device("cuda:0")

# layer output tolerance: relative L2 and max element error relative to RMS
REL_L2 = 2e-3
MAX_REL_RMS = 1e-2
# routing weights: absolute
W_ATOL = 2.0 ** -20


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def upload_weights(d):
    return {k: dev_u8(d[k]) for k in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")}


_PAGE = {}


def page_layer_weights():
    """Host and device weights of the page-shaped layer (hidden 6144, 384
    experts, intermediate 2048), shared by every workload that runs it."""
    if "host" not in _PAGE:
        cfg = workloads.CONFIGS["verify_t8"]
        say("generating page-shaped layer weights (%.2f GB)" % (cfg.E * cfg.expert_bytes() / 1e9))
        host = workloads.all_weights(cfg, 0)
        _PAGE["host"] = host
        _PAGE["dev"] = upload_weights(host)
        torch.cuda.synchronize()
    return _PAGE["host"], _PAGE["dev"]


def tol_check(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    rms = np.sqrt(np.mean(want ** 2))
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    mx = np.abs(got - want).max() / max(rms, 1e-300) if got.size else 0.0
    say("  %s: rel-L2 %.3g, max|d|/RMS %.3g" % (what, rel, mx))
    assert rel <= REL_L2, "%s: rel-L2 %.3g > %.3g" % (what, rel, REL_L2)
    assert mx <= MAX_REL_RMS, "%s: max|d|/RMS %.3g > %.3g" % (what, mx, MAX_REL_RMS)
    return rel, mx


def bf16_ulp_diff(a_bits, b_bits):
    """|a - b| in bf16 ulps for finite values (sign-magnitude to ordinal)."""
    def ordv(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(ordv(a_bits) - ordv(b_bits))


def run_layer(cfg, x_bits, logits, wdev):
    import mxfp4_moe_expert_route_amd as mm
    x = dev_bf16(x_bits)
    lg = torch.from_numpy(logits).to(DEV)
    b = mm.moe_mxfp4_layer(x, lg, cfg.k, wdev["w13_codes"], wdev["w13_scales"],
                           wdev["w2_codes"], wdev["w2_scales"])
    torch.cuda.synchronize()
    return b


def check_layer(cfg, x_bits, logits, whost, wdev, tokens=None, check_h=True):
    """Run the GPU layer and compare with the oracle: ids and lists bit-exact
    over every token, weights within W_ATOL, and out / h / y on `tokens`
    (all when None) within the stated tolerances."""
    b = run_layer(cfg, x_bits, logits, wdev)
    ref = olayer.layer_forward(x_bits, logits, whost["w13_codes"], whost["w13_scales"],
                               whost["w2_codes"], whost["w2_scales"], cfg.k, tokens=tokens)
    ids = b.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), "routing ids differ"
    w = b.topk_w.cpu().numpy()
    assert np.abs(w.astype(np.float64) - ref["w"]).max() <= W_ATOL, "routing weights differ"
    lists = operm.permute(ref["ids"], cfg.E)
    for key in ("counts", "offsets", "sorted_pairs", "pair_to_row"):
        assert np.array_equal(getattr(b, key).cpu().numpy(), lists[key]), key + " differs"
    tok = ref["tok"]
    out = b.out.cpu().numpy()[tok]
    res = tol_check(out, ref["out"], "%s out (%d tokens)" % (cfg.name, len(tok)))
    if check_h and len(tok):
        p2r = lists["pair_to_row"].reshape(cfg.T, cfg.k)[tok]          # [n, k]
        h = host_bits(b.h)[p2r]                                          # [n, k, I]
        d = bf16_ulp_diff(h, ref["h_bits"])
        say("  h: %.4f%% differ, %.4f%% by more than 1 ulp"
            % (100.0 * (d > 0).mean(), 100.0 * (d > 1).mean()))
        # h is rounded to bf16 on both sides from differently accumulated
        # sums: a rounding flip costs one ulp (large next to RMS for the
        # largest elements), and elements near zero come from cancelling sums
        # where fp32 and fp64 accumulation differ by many ulps of a small
        # value.  Per element: within max(1 ulp, 1e-2 RMS); overall: rel-L2
        # and the fraction beyond one ulp.
        assert (d > 1).mean() <= 1e-3, "h: too many elements off by more than 1 bf16 ulp"
        hg = omx.bf16_bits_to_f64(h)
        hr = omx.bf16_bits_to_f64(ref["h_bits"])
        rms = np.sqrt(np.mean(hr ** 2))
        _, ex = np.frexp(np.where(hr != 0, np.abs(hr), 1.0))
        ulp = np.ldexp(1.0, (ex - 1 - 7).astype(np.int32))
        assert np.all(np.abs(hg - hr) <= np.maximum(ulp, 1e-2 * rms)), "h element out of bound"
        rel = np.linalg.norm(hg - hr) / np.linalg.norm(hr)
        say("  %s h: rel-L2 %.3g" % (cfg.name, rel))
        assert rel <= REL_L2
        y = b.y.cpu().numpy()[p2r]
        tol_check(y, ref["y"], "%s y" % cfg.name)
    return b, ref, res
