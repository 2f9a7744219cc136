"""GPU parity of the whole layer (route -> permute -> gate/up+SwiGLU -> down
-> combine) against the oracle.

Small shapes are compared element by element over every token; they span
several tiles of every kernel and ragged tails.  The page-shaped workloads
(hidden 6144, 384 experts, top-8, intermediate 2048) run in full on the GPU
in the same launch configuration as the benchmark; routing and the
permutation lists are checked over every token, the layer output, h and y on
a sample of tokens the oracle evaluates one by one."""

import numpy as np
import pytest
import torch

import workloads
from _gpu import check_layer, page_layer_weights, say, upload_weights, run_layer

pytestmark = pytest.mark.gpu

SMALL = [
    # name, T, H, I, E, k
    ("tiny_t16", None),
    ("ragged_a", (37, 512, 256, 16, 4)),       # several n-tiles, rows per expert ~9
    ("ragged_b", (333, 256, 96, 8, 3)),        # rows per expert ~125 -> multi-subtile tiles
    ("one_tok", (1, 256, 128, 64, 8)),
    ("k_eq_e", (5, 128, 64, 4, 4)),            # every token picks every expert
    ("k1", (40, 192, 160, 12, 1)),             # I not a multiple of 64
    ("min_dims", (9, 32, 32, 3, 2)),           # one MX block per row
    ("many_e", (64, 256, 64, 1024, 32)),       # most experts empty
    ("wide_k", (300, 2048, 512, 32, 8)),
    ("fused_e960", (16, 256, 64, 960, 32)),   # routing and grouping fused (T <= 16), largest E
    ("wide_h16384", (4, 16384, 64, 4, 2)),     # largest H: 128 KB of scales in the streaming kernel
]

# experts with at least this many rows take the dense kernel (192-row items),
# the others the streaming kernels (16-row items)
DENSE_MIN_ROWS = 33

# shapes that take the LDS-tiled dense kernel (H, I multiples of 512, many
# rows per expert): one tile per expert, several tiles per expert, and a
# skewed mix where only the popular experts are dense
DENSE = [
    ("dense_one_tile", (300, 512, 512, 8, 4), "uniform"),
    ("dense_two_tiles", (700, 512, 1024, 4, 2), "uniform"),
    ("dense_mixed_zipf", (256, 1024, 512, 64, 8), "zipf"),
    # one expert: 192 + 8 rows, so the second m-tile leaves some waves without
    # token rows; 192 + 20 rows, a partial subtile for every wave
    ("dense_tail_8", (200, 512, 512, 1, 1), "uniform"),
    ("dense_tail_20", (212, 1024, 512, 1, 1), "uniform"),
    # 1024 rows per expert: 768 gate/up and 384 down items, so workgroups run
    # several items back to back (full m-tiles and 64-row last ones)
    ("dense_many_items", (4096, 512, 512, 32, 8), "uniform"),
    # three scale chunks per gate/up item (an odd count above one), and the
    # largest hidden size the decode kernel also takes
    ("dense_odd_chunks", (400, 1536, 512, 4, 2), "uniform"),
    ("dense_h8192", (1024, 8192, 1024, 8, 2), "uniform"),
]

# shapes that take the persistent decode kernel (H, I multiples of 2048, at
# most 16 rows per expert on average): a single token, experts split into
# several 16-row tiles by skewed routing, and enough units that each
# workgroup's run crosses several units and tiles.  decode_zipf_tiles also
# launches the dense kernel, which takes its two experts of 34 and 51 rows;
# decode_zipf_deep (fewer than 8 rows per touched expert: no dense launch)
# leaves an expert of 54 rows, four 16-row tiles, to the decode kernel;
# decode_h8192 runs gate/up at the largest K the kernel takes (8192),
# with experts of 17..21 rows in two tiles.
DECODE = [
    ("decode_one_tok", (1, 2048, 2048, 8, 4), "uniform"),
    ("decode_zipf_tiles", (64, 2048, 2048, 16, 2), "zipf"),
    ("decode_runs", (64, 2048, 2048, 32, 8), "uniform"),
    ("decode_zipf_deep", (64, 2048, 2048, 32, 2), "zipf"),
    ("decode_h8192", (32, 8192, 2048, 24, 4), "zipf"),
]


@pytest.fixture(scope="module")
def mm():
    import mxfp4_moe_expert_route_amd as m
    m._lib.lib()
    return m


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
def test_layer_small_every_token(mm, name, shape):
    if shape is None:
        cfg = workloads.CONFIGS[name]
    else:
        T, H, I, E, k = shape
        cfg = workloads.custom_config(name, 500 + SMALL.index((name, shape)), T, H, I, E, k)
    say("layer", name, cfg)
    d = workloads.layer_inputs(cfg, 0)
    check_layer(cfg, d["x_bits"], d["logits"], d, upload_weights(d))


def test_layer_fused_routing_ties(mm):
    """Up to 16 tokens are routed and grouped by one fused workgroup: integer
    logits (many ties), -0.0 next to +0.0 and NaN rows give the oracle's ids
    and lists bit for bit."""
    cfg = workloads.custom_config("fused_ties", 603, 12, 256, 64, 40, 6)
    say("layer", cfg.name, cfg)
    d = workloads.layer_inputs(cfg, 0)
    rng = np.random.default_rng(603)
    lg = rng.integers(-3, 4, size=(cfg.T, cfg.E)).astype(np.float32)
    lg[0, 5], lg[0, 6] = -0.0, 0.0
    lg[1, :] = np.nan
    lg[1, 7] = 1.0
    lg[2, 3] = np.nan
    check_layer(cfg, d["x_bits"], lg, d, upload_weights(d))


@pytest.mark.parametrize("name,shape,routing", DENSE, ids=[d[0] for d in DENSE])
def test_layer_dense_path_every_token(mm, name, shape, routing):
    T, H, I, E, k = shape
    cfg = workloads.custom_config(name, 700 + [d[0] for d in DENSE].index(name), T, H, I, E, k,
                                  routing=routing)
    say("layer", name, cfg)
    d = workloads.layer_inputs(cfg, 0)
    b, ref, _ = check_layer(cfg, d["x_bits"], d["logits"], d, upload_weights(d))
    counts = b.counts.cpu().numpy()
    say("  rows per expert: min %d max %d" % (counts.min(), counts.max()))
    assert counts.max() >= DENSE_MIN_ROWS            # at least one expert takes the dense kernel


@pytest.mark.parametrize("name,shape,routing", DECODE, ids=[d[0] for d in DECODE])
def test_layer_decode_path_every_token(mm, name, shape, routing):
    T, H, I, E, k = shape
    cfg = workloads.custom_config(name, 800 + [d[0] for d in DECODE].index(name), T, H, I, E, k,
                                  routing=routing)
    say("layer", name, cfg)
    d = workloads.layer_inputs(cfg, 0)
    b, ref, _ = check_layer(cfg, d["x_bits"], d["logits"], d, upload_weights(d))
    counts = b.counts.cpu().numpy()
    say("  rows per expert: min %d max %d" % (counts.min(), counts.max()))
    if name == "decode_h8192":
        assert counts.max() > 16                     # an expert in two tiles


def test_layer_is_deterministic(mm):
    cfg = workloads.custom_config("det", 601, 100, 512, 256, 32, 8)
    d = workloads.layer_inputs(cfg, 0)
    w = upload_weights(d)
    a = run_layer(cfg, d["x_bits"], d["logits"], w).out.clone()
    b = run_layer(cfg, d["x_bits"], d["logits"], w).out.clone()
    assert torch.equal(a, b)


def test_layer_skewed_routing_small(mm):
    cfg = workloads.custom_config("zipf_small", 602, 256, 256, 128, 64, 8, routing="zipf")
    d = workloads.layer_inputs(cfg, 0)
    b, ref, _ = check_layer(cfg, d["x_bits"], d["logits"], d, upload_weights(d))
    counts = b.counts.cpu().numpy()
    say("  zipf small: max rows/expert %d, mean %.1f" % (counts.max(), counts.mean()))
    assert counts.max() > 4 * counts.mean()


def sample_tokens(cfg, ids, n, seed=0):
    """n tokens: the first, the last, one routed to the most loaded expert,
    the rest random."""
    rng = np.random.default_rng(seed)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    hot = int(np.nonzero((ids == counts.argmax()).any(1))[0][0])
    pick = [0, cfg.T - 1, hot] + list(rng.choice(cfg.T, size=max(0, n - 3), replace=False))
    return np.array(sorted(set(int(p) for p in pick)))


@pytest.mark.parametrize("name,n", [("verify_t8", 8), ("verify_t64", 4), ("zipf_t512", 4),
                                    ("prefill_t8192", 4)])
def test_layer_page_shaped_sampled(mm, name, n):
    cfg = workloads.CONFIGS[name]
    whost, wdev = page_layer_weights()
    x = workloads.gen_x_bits(cfg, 0)
    logits = workloads.gen_logits(cfg, x, 0)
    from oracle import route as oroute
    ids, _ = oroute.route_topk(logits, cfg.k)
    tok = sample_tokens(cfg, ids, n) if n < cfg.T else None
    say("layer", name, "sampled tokens", tok)
    b, ref, _ = check_layer(cfg, x, logits, whost, wdev, tokens=tok)
    touched = int((b.counts.cpu().numpy() > 0).sum())
    say("  %s: touched experts %d" % (name, touched))


@pytest.mark.parametrize("name", ["verify_t64", "zipf_t512", "prefill_t8192"])
def test_page_shaped_every_block_written_and_sampled(mm, name):
    """At full size, in the benchmark's launch configuration: every element of
    h, y and the output is written (the buffers start as NaN), and one element
    of every work item of every kernel is checked against the oracle:
      h    every block of an expert's rows x 128 columns (gate/up items: 192
           token rows for experts with at least 33 rows, 16 for the others, by
           128 gate columns with their up columns);
      y    every block of those rows x 256 output features (down items), from
           the GPU's own h row;
      out  every token x 2048 columns (combine items), from the GPU's y rows.
    A skipped, repeated or misplaced item of any kernel shows."""
    from oracle import layer as olayer, mx as omx
    from oracle import permute as operm, route as oroute
    from _gpu import dev_bf16, bf16_ulp_diff
    cfg = workloads.CONFIGS[name]
    whost, wdev = page_layer_weights()
    x_bits = workloads.gen_x_bits(cfg, 0)
    logits = workloads.gen_logits(cfg, x_bits, 0)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    x = dev_bf16(x_bits)
    lg = torch.from_numpy(logits).to("cuda")
    ids_d, w_d, counts_d, offs_d, sp_d, p2r_d = mm.moe_route_permute(lg, k)
    h = torch.full((T * k, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mm.moe_mxfp4_gate_up_swiglu(x, sp_d, offs_d, k, wdev["w13_codes"], wdev["w13_scales"], h=h)
    mm.moe_mxfp4_down(h, offs_d, k, wdev["w2_codes"], wdev["w2_scales"], y=y)
    mm.moe_combine(y, w_d, p2r_d, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(h).all()), "h has unwritten (NaN) elements"
    assert bool(torch.isfinite(y).all()), "y has unwritten (NaN) elements"
    assert bool(torch.isfinite(out).all()), "out has unwritten (NaN) elements"

    ids, _ = oroute.route_topk(logits, k)
    lists = operm.permute(ids, E)
    assert np.array_equal(offs_d.cpu().numpy(), lists["offsets"])
    assert np.array_equal(p2r_d.cpu().numpy(), lists["pair_to_row"])
    offsets, sorted_pairs = lists["offsets"], lists["sorted_pairs"]
    rng = np.random.default_rng(7)
    rows, cols = [], []
    for e in range(E):
        n_e = int(offsets[e + 1] - offsets[e])
        blk = 192 if n_e >= DENSE_MIN_ROWS else 16
        for r0 in range(0, n_e, blk):
            nr = min(blk, n_e - r0)
            for c0 in range(0, I, 128):
                rows.append(int(offsets[e]) + r0 + int(rng.integers(nr)))
                cols.append(c0 + int(rng.integers(128)))
    rows, cols = np.array(rows), np.array(cols)
    hg_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)[rows, cols]
    experts = np.searchsorted(offsets, rows, side="right") - 1
    tokens = sorted_pairs[rows] // k
    X = omx.bf16_bits_to_f64(x_bits[tokens])
    hr_bits = np.empty(len(rows), np.uint16)
    for i in range(len(rows)):
        e, c = experts[i], cols[i]
        sel = [c, I + c]
        hr_bits[i] = olayer.gate_up_swiglu(X[i:i + 1], whost["w13_codes"][e][sel],
                                           whost["w13_scales"][e][sel])[0, 0]
    d = bf16_ulp_diff(hg_bits, hr_bits)
    hg, hr = omx.bf16_bits_to_f64(hg_bits), omx.bf16_bits_to_f64(hr_bits)
    rms = np.sqrt(np.mean(hr ** 2))
    _, ex = np.frexp(np.where(hr != 0, np.abs(hr), 1.0))
    ulp = np.ldexp(1.0, (ex - 1 - 7).astype(np.int32))
    say("  %s: %d sampled h elements (one per block), %.3f%% differ, max %d ulp"
        % (name, len(rows), 100.0 * (d > 0).mean(), int(d.max())))
    assert np.all(np.abs(hg - hr) <= np.maximum(ulp, 1e-2 * rms)), "h element out of bound"
    assert (d > 1).mean() <= 1e-3

    # y: one element of every down work item, an expert's block of rows (192
    # or 16, as above) by 256 output features, against the oracle's down row
    # applied to the GPU's own h row in float64.  fp32 accumulation of I
    # products is within I * 2^-24 of their absolute sum; the bound is twice
    # that, far below what a misplaced or stale item would show.
    h_all = h.view(torch.int16).cpu().numpy().view(np.uint16)
    y_all = y.cpu().numpy()
    rows, cols = [], []
    for e in range(E):
        n_e = int(offsets[e + 1] - offsets[e])
        blk = 192 if n_e >= DENSE_MIN_ROWS else 16
        for r0 in range(0, n_e, blk):
            nr = min(blk, n_e - r0)
            for c0 in range(0, H, 256):
                rows.append(int(offsets[e]) + r0 + int(rng.integers(nr)))
                cols.append(c0 + int(rng.integers(256)))
    rows, cols = np.array(rows), np.array(cols)
    experts = np.searchsorted(offsets, rows, side="right") - 1
    worst = 0.0
    for c0 in range(0, len(rows), 2048):
        r, c, e = rows[c0:c0 + 2048], cols[c0:c0 + 2048], experts[c0:c0 + 2048]
        W = omx.unpack(whost["w2_codes"][e, c], whost["w2_scales"][e, c])        # [n, I]
        hv = omx.bf16_bits_to_f64(h_all[r])                                      # [n, I]
        exact = (W * hv).sum(1)
        mag = np.abs(W * hv).sum(1)
        err = np.abs(y_all[r, c].astype(np.float64) - exact)
        assert np.all(err <= 2.0 * I * 2.0 ** -24 * mag + 1e-30), "y element out of bound"
        worst = max(worst, float((err / np.maximum(mag, 1e-300)).max()))
    say("  %s: %d sampled y elements (one per down item), worst |d| / sum|h w| %.3g"
        % (name, len(rows), worst))

    # out: one element of every combine item (a token by 2048 columns),
    # against the slot-ordered sum of the GPU's own y rows in float64
    w_h = w_d.cpu().numpy().astype(np.float64)
    p2r = lists["pair_to_row"].reshape(T, k)
    out_all = out.cpu().numpy()
    toks = np.repeat(np.arange(T), (H + 2047) // 2048)
    cb = np.tile(np.arange(0, H, 2048), T)
    cols = cb + rng.integers(0, np.minimum(2048, H - cb))
    terms = w_h[toks] * y_all[p2r[toks], cols[:, None]].astype(np.float64)   # [n, k]
    err = np.abs(out_all[toks, cols] - terms.sum(1))
    assert np.all(err <= 2.0 * k * 2.0 ** -24 * np.abs(terms).sum(1) + 1e-30), \
        "out element out of bound"
    say("  %s: %d sampled out elements (one per combine item)" % (name, len(toks)))
