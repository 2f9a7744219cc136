"""The seeded input generator: determinism, per-expert regeneration, shapes
and distributions of the configured workloads."""

import numpy as np
import torch

import workloads


def test_configs_use_the_pages_constants(golden):
    c = {r[0]: int(r[1]) for r in golden("page_constants.txt")}
    for name in ("verify_t8", "verify_t64", "zipf_t512", "prefill_t8192"):
        cfg = workloads.CONFIGS[name]
        assert (cfg.H, cfg.E, cfg.k) == (c["hidden"], c["experts"], c["topk"])
        assert cfg.T % c["verify_block"] == 0
    assert workloads.CONFIGS["verify_t8"].T == c["verify_block"]
    assert workloads.CONFIGS["verify_t8"].expert_bytes() == 20054016


def test_x_rounding_matches_torch_bf16():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000).astype(np.float32)
    ours = workloads.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generation_is_deterministic_and_per_expert():
    cfg = workloads.CONFIGS["tiny_t16"]
    a = workloads.layer_inputs(cfg, 0)
    b = workloads.layer_inputs(cfg, 0)
    for key in a:
        assert np.array_equal(a[key], b[key])
    lazy = workloads.lazy_weights(cfg, 0)
    for e in (0, 5, 7):
        for key in lazy:
            assert np.array_equal(lazy[key][e], a[key][e])
    c = workloads.layer_inputs(cfg, 1)
    assert not np.array_equal(a["w13_codes"], c["w13_codes"])


def test_value_distributions():
    cfg = workloads.CONFIGS["tiny_t16"]
    d = workloads.layer_inputs(cfg, 0)
    s = d["w13_scales"]
    assert s.min() == cfg.exp_lo and s.max() == cfg.exp_hi
    nib = np.concatenate([(d["w13_codes"] & 15).ravel(), (d["w13_codes"] >> 4).ravel()])
    hist = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(hist - 1 / 16) < 0.01)
    x = workloads.bf16_bits_as_f32(d["x_bits"])
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1) < 0.1


def test_zipf_bias_skews_routing():
    cfg = workloads.custom_config("z", 77, 512, 256, 32, 384, 8, routing="zipf")
    x = workloads.gen_x_bits(cfg, 0)
    l = workloads.gen_logits(cfg, x, 0)
    top = np.argsort(-l, axis=1)[:, :8]
    counts = np.bincount(top.ravel(), minlength=384)
    assert counts.max() > 10 * counts.mean()
