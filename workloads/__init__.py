"""Seeded synthetic inputs for the MXFP4 MoE expert layer.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic.  Both the oracle checks and the HIP path consume what
it produces.  Every tensor has its own numpy stream,
SeedSequence([seed, config id, tensor id(, expert)]), so any single expert's
weights can be regenerated on its own.

Recipe (shapes from the pages: hidden 6144 in the "MiMo-V2.5-Pro-FP4-DFlash"
model card §4 "Model Summary"; 384 experts, top-8 in the nxbn.cn article
"架构设计与配置详解"; MXFP4 block 32 in the model card §2; 8 tokens per
verify step from the DFlash block cap in §3.  The expert intermediate size
2048 is not on the pages and is an assumption):
  x          ~N(0,1) drawn in fp32, rounded to bf16 (RNE)
  W_router   ~N(0, 0.02) fp32 (0.02 read as the standard deviation)
  logits     fp32( fp64(x) . fp64(W_router)^T [+ b] ), rounded once
  b (zipf)   b_e = ln p_rank(e), p_r proportional to r**-s over r = 1..E,
             rank(e) a seeded permutation of the experts
  codes      uniform random bytes (two independent uniform 4-bit codes each)
  scales     uniform integers in [exp_lo, exp_hi]
"""

from dataclasses import dataclass, replace

import numpy as np

# tensor ids of the per-tensor streams
_T_X, _T_ROUTER, _T_BIAS = 1, 2, 3
_T_W13C, _T_W13S, _T_W2C, _T_W2S = 10, 11, 12, 13


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    T: int
    H: int
    I: int
    E: int
    k: int
    exp_lo: int
    exp_hi: int
    routing: str = "uniform"     # "uniform" | "zipf"
    zipf_s: float = 1.1
    router_std: float = 0.02
    layer_id: int = -1           # seeds weights and router; -1: same as cfg_id

    @property
    def lid(self):
        return self.cfg_id if self.layer_id < 0 else self.layer_id

    @property
    def R(self):
        return self.T * self.k

    def with_tokens(self, T):
        return replace(self, T=T)

    def expert_bytes(self):
        """MXFP4 bytes of one expert: W13 codes+scales and W2 codes+scales."""
        H, I = self.H, self.I
        return 2 * I * H // 2 + 2 * I * H // 32 + H * I // 2 + H * I // 32


CONFIGS = {
    # hidden 256, 8 experts, top-2, intermediate 128, 16 tokens; seed 0
    "tiny_t16": LayerConfig("tiny_t16", 0, 16, 256, 128, 8, 2, 119, 123, layer_id=0),
    # page-shaped layer (layer id 1), one sequence's 8-token verify block
    "verify_t8": LayerConfig("verify_t8", 1, 8, 6144, 2048, 384, 8, 118, 124, layer_id=1),
    # same layer, 8 sequences x 8-token blocks
    "verify_t64": LayerConfig("verify_t64", 2, 64, 6144, 2048, 384, 8, 118, 124, layer_id=1),
    # same layer, 64 sequences x 8 tokens, Zipf(1.1) expert popularity
    "zipf_t512": LayerConfig("zipf_t512", 3, 512, 6144, 2048, 384, 8, 118, 124,
                             routing="zipf", layer_id=1),
    # same layer, prefill-like: 8192 tokens, dense expert GEMMs
    "prefill_t8192": LayerConfig("prefill_t8192", 4, 8192, 6144, 2048, 384, 8,
                                 118, 124, layer_id=1),
}


def custom_config(name, cfg_id, T, H, I, E, k, exp_lo=118, exp_hi=124,
                  routing="uniform"):
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    return LayerConfig(name, cfg_id, T, H, I, E, k, exp_lo, exp_hi, routing)


def _rng(seed, *ids):
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(i) for i in ids]))


def _random_bytes(rng, n):
    """n uniform random bytes (n % 8 == 0) from the stream's raw 64-bit words."""
    if n % 8:
        raise ValueError("byte count must be a multiple of 8")
    return rng.bit_generator.random_raw(n // 8).view(np.uint8)


def f32_to_bf16_bits(v):
    """Round fp32 values (finite) to bf16 bit patterns, nearest-even."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_as_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_x_bits(cfg, seed=0):
    x = _rng(seed, cfg.cfg_id, _T_X).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def gen_router(cfg, seed=0):
    r = _rng(seed, cfg.lid, _T_ROUTER)
    return r.normal(0.0, cfg.router_std, size=(cfg.E, cfg.H)).astype(np.float32)


def gen_bias(cfg, seed=0):
    """fp64 [E] logit bias: zeros for uniform routing, Zipf log-popularity else."""
    if cfg.routing == "uniform":
        return np.zeros(cfg.E, np.float64)
    if cfg.routing != "zipf":
        raise ValueError("unknown routing " + cfg.routing)
    r = _rng(seed, cfg.cfg_id, _T_BIAS)
    rank = r.permutation(cfg.E)                  # rank[e] in 0..E-1
    p = np.arange(1, cfg.E + 1, dtype=np.float64) ** (-cfg.zipf_s)
    p /= p.sum()
    return np.log(p[rank])


def gen_logits(cfg, x_bits, seed=0):
    W = gen_router(cfg, seed).astype(np.float64)
    x = bf16_bits_as_f32(x_bits).astype(np.float64)
    return (x @ W.T + gen_bias(cfg, seed)[None, :]).astype(np.float32)


def expert_weights(cfg, e, seed=0):
    """(w13_codes [2I,H/2], w13_scales [2I,H/32], w2_codes [H,I/2], w2_scales [H,I/32])
    for expert e, all uint8."""
    H, I = cfg.H, cfg.I
    c13 = _random_bytes(_rng(seed, cfg.lid, _T_W13C, e), 2 * I * H // 2)
    s13 = _rng(seed, cfg.lid, _T_W13S, e).integers(
        cfg.exp_lo, cfg.exp_hi + 1, size=2 * I * H // 32, dtype=np.uint8)
    c2 = _random_bytes(_rng(seed, cfg.lid, _T_W2C, e), H * I // 2)
    s2 = _rng(seed, cfg.lid, _T_W2S, e).integers(
        cfg.exp_lo, cfg.exp_hi + 1, size=H * I // 32, dtype=np.uint8)
    return (c13.reshape(2 * I, H // 2), s13.reshape(2 * I, H // 32),
            c2.reshape(H, I // 2), s2.reshape(H, I // 32))


def all_weights(cfg, seed=0, out=None):
    """All experts stacked: dict of uint8 arrays w13_codes [E,2I,H/2],
    w13_scales [E,2I,H/32], w2_codes [E,H,I/2], w2_scales [E,H,I/32].
    `out` may supply preallocated arrays (e.g. pinned host memory views)."""
    H, I, E = cfg.H, cfg.I, cfg.E
    shapes = {"w13_codes": (E, 2 * I, H // 2), "w13_scales": (E, 2 * I, H // 32),
              "w2_codes": (E, H, I // 2), "w2_scales": (E, H, I // 32)}
    if out is None:
        out = {k: np.empty(s, np.uint8) for k, s in shapes.items()}
    for e in range(E):
        c13, s13, c2, s2 = expert_weights(cfg, e, seed)
        out["w13_codes"][e] = c13
        out["w13_scales"][e] = s13
        out["w2_codes"][e] = c2
        out["w2_scales"][e] = s2
    return out


class LazyExperts:
    """Index-by-expert view that regenerates one expert on demand (for the
    oracle at full size without materialising every expert)."""

    def __init__(self, cfg, part, seed=0):
        self.cfg, self.part, self.seed = cfg, part, seed
        self._idx = {"w13_codes": 0, "w13_scales": 1, "w2_codes": 2, "w2_scales": 3}[part]

    def __len__(self):
        return self.cfg.E

    _cache = {}

    def __getitem__(self, e):
        key = (self.cfg.lid, self.cfg.H, self.cfg.I, self.cfg.exp_lo, self.cfg.exp_hi, self.seed,
               int(e))
        if key not in LazyExperts._cache:
            LazyExperts._cache.clear()             # keep one expert resident
            LazyExperts._cache[key] = expert_weights(self.cfg, int(e), self.seed)
        return LazyExperts._cache[key][self._idx]


def lazy_weights(cfg, seed=0):
    return {p: LazyExperts(cfg, p, seed)
            for p in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")}


def layer_inputs(cfg, seed=0, weights=True):
    """x_bits, logits and (optionally) all expert weights for one config."""
    x = gen_x_bits(cfg, seed)
    d = {"x_bits": x, "logits": gen_logits(cfg, x, seed)}
    if weights:
        d.update(all_weights(cfg, seed))
    return d


# ---- drafted blocks for the verification step (a "next" row) -------------

VERIFY_VOCAB = 152064      # reading: the pages give only a mask token id of 151669


def gen_verify_inputs(B, L=8, V=VERIFY_VOCAB, seed=0, logit_std=3.0, draft_noise=0.35):
    """Synthetic inputs of B drafted blocks: backbone logits [B, L+1, V] ~
    N(0, logit_std^2); drafter probabilities [B, L, V] = softmax of the
    backbone logits plus N(0, draft_noise^2) (per-token acceptance about
    0.88, about 4.6 of 8 tokens accepted on average); drafted tokens drawn from
    the drafter's probabilities; uniforms in [0, 1).  All float32 / int32."""
    r = _rng(seed, 77, B, L, V)
    target = r.normal(0.0, logit_std, size=(B, L + 1, V)).astype(np.float32)
    noisy = target[:, :L, :].astype(np.float64) + r.normal(0.0, draft_noise, size=(B, L, V))
    noisy -= noisy.max(axis=2, keepdims=True)
    q = np.exp(noisy)
    q /= q.sum(axis=2, keepdims=True)
    draft = q.astype(np.float32)
    c = np.cumsum(q, axis=2)
    pick = r.random((B, L, 1)) * c[:, :, -1:]
    tokens = np.minimum((c <= pick).sum(axis=2), V - 1).astype(np.int32)
    uniforms = np.minimum(r.random((B, L + 1)), 1.0 - 2.0 ** -24).astype(np.float32)
    return target, draft, tokens, uniforms
