"""Pins of the oracle's layer: textbook special case, pure-Python brute force,
and invariances a mistake in indexing or combining would break."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as olayer
from oracle import mx


def bitfield_table():
    out = []
    for c in range(16):
        s, E, M = (c >> 3) & 1, (c >> 1) & 3, c & 1
        v = 0.5 * M if E == 0 else 2.0 ** (E - 1) * (1 + M / 2)
        out.append(-v if s else v)
    return np.array(out)


def dequant_indep(codes, scales):
    """Dequantise from the bit-field definition (independent of oracle.mx)."""
    codes = np.asarray(codes)
    rows, half = codes.shape
    el = np.stack([codes & 15, codes >> 4], -1).reshape(rows, half * 2)
    v = bitfield_table()[el]
    s = np.exp2(np.asarray(scales, np.float64) - 127)
    return v * np.repeat(s, 32, axis=1)


def small_layer(T, H, I, E, k, seed, exp=(118, 124)):
    cfg = workloads.custom_config("t", 900 + seed, T, H, I, E, k, *exp)
    d = workloads.layer_inputs(cfg, seed)
    return cfg, d


def run(d, k, tokens=None):
    return olayer.layer_forward(d["x_bits"], d["logits"], d["w13_codes"], d["w13_scales"],
                                d["w2_codes"], d["w2_scales"], k, tokens=tokens)


def test_single_expert_is_a_textbook_swiglu_ffn():
    cfg, d = small_layer(T=5, H=64, I=32, E=1, k=1, seed=1)
    r = run(d, 1)
    x = torch.from_numpy(workloads.bf16_bits_as_f32(d["x_bits"]).astype(np.float64))
    W13 = torch.from_numpy(dequant_indep(d["w13_codes"][0], d["w13_scales"][0]))
    W2 = torch.from_numpy(dequant_indep(d["w2_codes"][0], d["w2_scales"][0]))
    g = x @ W13[:32].T
    u = x @ W13[32:].T
    a = torch.nn.functional.silu(g) * u
    h_bits = mx.to_bf16_bits(a.numpy())              # bf16 rounding is pinned separately
    assert np.array_equal(r["h_bits"][:, 0], h_bits)
    y = (torch.from_numpy(mx.bf16_bits_to_f64(h_bits)) @ W2.T).numpy()
    assert np.allclose(r["out"], y, rtol=2e-7, atol=0)
    assert np.all(r["w"] == 1.0) and np.all(r["ids"] == 0)


def test_brute_force_python_loops_on_tiny_config():
    cfg = workloads.CONFIGS["tiny_t16"]
    d = workloads.layer_inputs(cfg, 0)
    toks = [3, 11]
    r = run(d, cfg.k, tokens=toks)
    tab = bitfield_table()

    def wval(codes, scales, n, kk):
        byte = int(codes[n, kk // 2])
        c = byte & 15 if kk % 2 == 0 else byte >> 4
        return tab[c] * 2.0 ** (int(scales[n, kk // 32]) - 127)

    xs = workloads.bf16_bits_as_f32(d["x_bits"]).astype(np.float64)
    for n_t, t in enumerate(toks):
        row = [float(v) for v in d["logits"][t]]
        order = sorted(range(cfg.E), key=lambda e: (-row[e], e))[:cfg.k]
        ex = [math.exp(row[e] - row[order[0]]) for e in order]
        wts = [v / sum(ex) for v in ex]
        assert list(r["ids"][t]) == order
        out = [0.0] * cfg.H
        for j, e in enumerate(order):
            c13, s13 = d["w13_codes"][e], d["w13_scales"][e]
            c2, s2 = d["w2_codes"][e], d["w2_scales"][e]
            h = []
            for i in range(cfg.I):
                g = sum(xs[t, kk] * wval(c13, s13, i, kk) for kk in range(cfg.H))
                u = sum(xs[t, kk] * wval(c13, s13, cfg.I + i, kk) for kk in range(cfg.H))
                h.append(g / (1 + math.exp(-g)) * u)
            hb = mx.to_bf16_bits(np.array(h))
            assert np.array_equal(r["h_bits"][n_t, j], hb)
            hv = mx.bf16_bits_to_f64(hb)
            for n in range(cfg.H):
                yv = sum(hv[i] * wval(c2, s2, n, i) for i in range(cfg.I))
                yv32 = float(np.float32(yv))
                assert abs(float(r["y"][n_t, j, n]) - yv32) <= 2 * abs(yv32) * 2 ** -24 + 1e-30
                out[n] += float(np.float32(wts[j])) * yv32
        assert np.allclose(r["out"][n_t], out, rtol=1e-6, atol=1e-6 * max(map(abs, out)))


def test_relabelling_experts_leaves_output_unchanged():
    cfg, d = small_layer(T=20, H=64, I=32, E=12, k=3, seed=2)
    perm = np.random.default_rng(5).permutation(cfg.E)          # new id of old expert e
    inv = np.argsort(perm)
    d2 = dict(d)
    d2["logits"] = d["logits"][:, inv]
    for key in ("w13_codes", "w13_scales", "w2_codes", "w2_scales"):
        d2[key] = d[key][inv]
    r1, r2 = run(d, cfg.k), run(d2, cfg.k)
    assert np.array_equal(perm[r1["ids"]], r2["ids"])
    assert np.array_equal(r1["out"], r2["out"])


def test_token_order_equivariance_and_sampling():
    cfg, d = small_layer(T=17, H=64, I=64, E=6, k=2, seed=3)
    r = run(d, cfg.k)
    p = np.random.default_rng(1).permutation(cfg.T)
    d2 = dict(d)
    d2["x_bits"], d2["logits"] = d["x_bits"][p], d["logits"][p]
    r2 = run(d2, cfg.k)
    assert np.array_equal(r2["out"], r["out"][p])
    sub = run(d, cfg.k, tokens=[9, 2, 16])
    assert np.array_equal(sub["out"], r["out"][[9, 2, 16]])


def test_zero_token_gives_zero_output():
    cfg, d = small_layer(T=4, H=64, I=32, E=4, k=2, seed=4)
    d["x_bits"][2] = 0
    r = run(d, cfg.k)
    assert np.all(r["out"][2] == 0) and np.any(r["out"][1] != 0)


def test_output_is_linear_in_the_routing_weights():
    """Swapping the top-2 logits of a token swaps its weights and keeps out
    equal to w0*y(e0) + w1*y(e1) with the per-expert outputs unchanged."""
    cfg, d = small_layer(T=6, H=64, I=32, E=5, k=2, seed=6)
    r = run(d, cfg.k)
    for t in range(cfg.T):
        y0 = r["y"][t, 0].astype(np.float64)
        y1 = r["y"][t, 1].astype(np.float64)
        w0, w1 = float(r["w"][t, 0]), float(r["w"][t, 1])
        assert np.allclose(r["out"][t], w0 * y0 + w1 * y1, rtol=1e-6, atol=1e-6)
        assert abs(w0 + w1 - 1) < 1e-6
