"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

One step = the whole layer (moe_route_permute (top-k routing and grouping by
expert) -> moe_mxfp4_gate_up_swiglu -> moe_mxfp4_down -> moe_combine) over one batch of
synthetic tokens, inputs resident in HBM.  Default workload: the page-shaped
layer (hidden 6144, 384 experts, top-8, intermediate 2048, MXFP4 block 32)
verifying one sequence's 8-token draft block.  Two copies of the expert
weights alternate between steps so the 256 MB last-level cache cannot serve
them.

Prints ONE JSON line on stdout; diagnostics go to stderr.
  value       tokens/s of the whole layer
  roofline    the gate/up contraction (the kernel that streams 2/3 of the
              weight bytes): algorithmic bytes per launch / its mean duration
              from HIP events recorded around it on its stream inside the
              timed region, against 8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same tokens
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 MoE layer tokens/s + effective weight GB/s (% HBM peak) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3
LLC_BYTES = 256 * 1024 * 1024                 # MI355X last-level (Infinity) cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Kernels that each entry point launches (a substring of the demangled name).
ENTRY_KERNELS = {
    "moe_mxfp4_gate_up_swiglu": ("k_decode<true>", "k_gate_up<", "k_dense<true>"),
    "moe_mxfp4_down": ("k_decode<false>", "k_down<", "k_dense<false>"),
}
# source file of each kernel family; every measurement also depends on the
# shared helpers and on the host code that picks the kernel
KERNEL_FILES = {"k_decode": "expert_decode.hip", "k_gate_up": "expert_stream.hip",
                "k_down": "expert_stream.hip", "k_dense": "expert_dense.hip"}
COMMON_FILES = ("common.hpp", "expert_stream.hip", "api.hip")


def kernel_sources(kernel_names):
    files = set(COMMON_FILES)
    for n in kernel_names:
        files.update(f for k, f in KERNEL_FILES.items() if k in n)
    return sorted(files)


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mxfp4_moe_expert_route_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when it is missing or was taken from another version of the kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("%s@%s" % (kernel, workload))
    if not rec or "sources" not in rec or \
            rec.get("source_hash") != kernel_source_hash(rec["sources"]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, x_bits, logits, whost, budget_s):
    """Time the oracle on growing token subsets until `budget_s` is spent."""
    from oracle import layer as olayer
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    done, elapsed = 0, 0.0
    step = max(1, min(cfg.T, 2))
    while done < cfg.T and elapsed < budget_s:
        tok = np.arange(done, min(cfg.T, done + step))
        t0 = time.perf_counter()
        olayer.layer_forward(x_bits, logits, whost["w13_codes"], whost["w13_scales"],
                             whost["w2_codes"], whost["w2_scales"], cfg.k, tokens=tok)
        elapsed += time.perf_counter() - t0
        done += len(tok)
    return {"value": done / elapsed, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d of %d tokens of %s, whole layer (routing of all tokens, float64 "
                      "dequantised expert FFNs, combine) with numpy on the host, %.1f s"
                      % (done, cfg.T, cfg.name, elapsed)}


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for fn in sorted(files):
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError("no *%s under %s" % (suffix, d))


def _algorithmic_bytes(cfg, counts):
    """Algorithmic HBM bytes of one call of each contraction entry point: the
    touched experts' weights, plus the layer input x read once by gate/up (the
    intermediates h and y could be fused away and are not counted)."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    touched = int((np.asarray(counts) > 0).sum())
    w13 = 2 * I * H // 2 + 2 * I * H // 32
    w2 = H * I // 2 + H * I // 32
    return {"moe_mxfp4_gate_up_swiglu": touched * w13 + T * H * 2,
            "moe_mxfp4_down": touched * w2, "touched": touched}


def summarize_profiles(args):
    """rocprofv3 output of bench.py runs -> the committed summaries.

    Prints a markdown table of the kernel-trace statistics and, given the two
    PMC runs (FETCH_SIZE, then WRITE_SIZE), stores in profiles/traffic.json the
    calibrated HBM bytes per call of each contraction entry point.  The
    counters are scaled by what they read for the largest weight clone
    (a plain copy kernel of known size) in the same run."""
    import workloads
    cfg = workloads.CONFIGS[args.config]
    out = ["# Kernel times and HBM traffic, %s workload (%d tokens, hidden %d, %d experts, "
           "top-%d, intermediate %d)" % (cfg.name, cfg.T, cfg.H, cfg.E, cfg.k, cfg.I), ""]
    if args.command:
        out += ["Command (from /tmp, `TMPDIR=/tmp`, on one MI355X):", "", "```",
                args.command, "```", ""]
    if args.stats_dir:
        rows = _csv_rows(_find_csv(args.stats_dir, "kernel_stats.csv"))
        out += ["| kernel | calls | average (us) | min (us) | max (us) | share |",
                "|---|---|---|---|---|---|"]
        for r in rows:
            name = r["Name"].replace("mxm::(anonymous namespace)::", "").replace(
                "void ", "").split("(")[0]
            out.append("| %s | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        out.append("")
    if args.fetch_dir and args.write_dir:
        known = cfg.E * 2 * cfg.I * cfg.H // 2          # the w13 codes clone
        per = {}
        names = {}
        factors = {}
        for ctr, d in (("FETCH_SIZE", args.fetch_dir), ("WRITE_SIZE", args.write_dir)):
            rows = [r for r in _csv_rows(_find_csv(d, "counter_collection.csv"))
                    if r["Counter_Name"] == ctr]
            copies = [float(r["Counter_Value"]) for r in rows
                      if "copyBuffer" in r["Kernel_Name"]]
            factors[ctr] = known / (max(copies) * 1024.0)
            for entry, pats in ENTRY_KERNELS.items():
                by_kernel = {}
                for r in rows:
                    if any(p in r["Kernel_Name"] for p in pats):
                        by_kernel.setdefault(r["Kernel_Name"], []).append(
                            float(r["Counter_Value"]))
                names.setdefault(entry, set()).update(by_kernel)
                per.setdefault(entry, {})[ctr] = sum(
                    np.mean(v) * 1024.0 * factors[ctr] for v in by_kernel.values())
        alg = _algorithmic_bytes(cfg, np.load(args.counts) if args.counts else
                                 np.full(cfg.E, 1))
        path = os.path.join(ROOT, "profiles", "traffic.json")
        db = json.load(open(path)) if os.path.exists(path) else {}
        out += ["Calibration: the largest weight clone copies %d B; FETCH_SIZE reads %.4g KiB "
                "for it (factor %.3f), WRITE_SIZE %.4g KiB (factor %.3f)."
                % (known, known / 1024.0 / factors["FETCH_SIZE"], factors["FETCH_SIZE"],
                   known / 1024.0 / factors["WRITE_SIZE"], factors["WRITE_SIZE"]), "",
                "| entry point | fetched (MB/call) | written (MB/call) | total (MB/call) | "
                "algorithmic (MB/call) | ratio |", "|---|---|---|---|---|---|"]
        for entry, v in per.items():
            tot = v["FETCH_SIZE"] + v["WRITE_SIZE"]
            out.append("| %s | %.1f | %.1f | %.1f | %.1f | %.3f |" % (
                entry, v["FETCH_SIZE"] / 1e6, v["WRITE_SIZE"] / 1e6, tot / 1e6,
                alg[entry] / 1e6, tot / alg[entry]))
            srcs = kernel_sources(names[entry])
            db["%s@%s" % (entry, cfg.name)] = {
                "sources": srcs, "source_hash": kernel_source_hash(srcs),
                "bytes_per_launch": int(round(tot)),
                "fetch_bytes": int(round(v["FETCH_SIZE"])),
                "write_bytes": int(round(v["WRITE_SIZE"])),
                "algorithmic_bytes": int(alg[entry]),
                "fetch_factor": round(factors["FETCH_SIZE"], 4),
                "write_factor": round(factors["WRITE_SIZE"], 4)}
        out.append("")
        with open(path, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
    print("\n".join(out))


def bench_router(args, cfg, torch, mm, workloads):
    """One JSON line for moe_router_topk on the workload's tokens: the fp32
    router weights [E, H] are read once per block of tokens, so at decode
    sizes the call streams them from HBM; above, fp32 FMAs bound it."""
    dev = torch.device("cuda:0")
    steps = args.steps or 200
    warmup = args.warmup if args.warmup is not None else 20
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    x = torch.from_numpy(workloads.gen_x_bits(cfg, 0).view(np.int16)).view(torch.bfloat16).to(dev)
    # enough copies of the router weights that together they are twice the
    # 256 MB last-level cache, used in turn, so each call reads its copy from HBM
    w0 = torch.from_numpy(workloads.gen_router(cfg, 0)).to(dev)
    ncopy = max(2, -(-2 * LLC_BYTES // (E * H * 4)))
    w = [w0] + [w0.clone() for _ in range(ncopy - 1)]
    bias = torch.from_numpy(workloads.gen_bias(cfg, 0).astype(np.float32)).to(dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(T, k, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        mm.moe_router_topk(x, w[i % ncopy], k, bias, logits, ids, tw)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        mm.moe_router_topk(x, w[i % ncopy], k, bias, logits, ids, tw)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = E * H * 4 + T * H * 2 + E * 4 + T * E * 4 + T * k * 8
    flops = 2.0 * T * E * H
    if flops / nbytes < FP32_VALU_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        ach = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4)}
    else:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(ach, 2), "peak": FP32_VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP32_VALU_PEAK_TFLOPS, 4)}
    roof.update({"kernel": "moe_router_topk", "algorithmic_bytes": nbytes,
                 "algorithmic_flops": flops, "mean_launch_ms": round(ms, 5), "traffic": None})
    print(json.dumps({
        "metric": "router projection + top-k tokens/s on 1 MI355X", "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " router", "tokens": T, "hidden": H, "experts": E,
                   "top_k": k, "router_weights": "f32 [E, H]", "parallelism": "none (1 GPU)"},
        "roofline": roof, "cpu_baseline": None}), flush=True)


def bench_verify(args, cfg, torch, mm, workloads):
    """One JSON line for dflash_verify_accept: T / 8 drafted blocks of 8 over
    the vocabulary.  Algorithmic bytes per block: the L + 1 rows of target
    logits, the drafter's row at the first rejected position, the drafter's
    probabilities at the L drafted tokens, the tokens, the uniforms and the
    two outputs.  The kernels read target row n a second time (from cache
    when it is still there); that re-read is not counted."""
    dev = torch.device("cuda:0")
    steps = args.steps or 200
    warmup = args.warmup if args.warmup is not None else 20
    L, V = 8, workloads.VERIFY_VOCAB
    B = max(1, cfg.T // L)
    if B > 64:
        print("bench.py: --verify runs workloads of up to 512 tokens (64 blocks)", file=sys.stderr)
        sys.exit(2)
    tg, dr, tk, u = workloads.gen_verify_inputs(B, L, V, 0)
    # enough copies of the inputs that together they are twice the last-level
    # cache, used in turn, so each call reads its inputs from HBM
    in0 = tuple(torch.from_numpy(a).to(dev) for a in (tg, dr, tk, u))
    set_bytes = sum(a.numel() * a.element_size() for a in in0)
    ncopy = max(2, -(-2 * LLC_BYTES // set_bytes))
    ins = [in0] + [tuple(a.clone() for a in in0) for _ in range(ncopy - 1)]
    n = torch.empty(B, dtype=torch.int32, device=dev)
    t = torch.empty(B, dtype=torch.int32, device=dev)
    ws = torch.empty(max(8, int(mm._lib.lib().dflash_verify_workspace_bytes(B, L, V))),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        mm.dflash_verify_accept(*ins[i % ncopy], n, t, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        mm.dflash_verify_accept(*ins[i % ncopy], n, t, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = B * ((L + 2) * V * 4 + L * 4 + L * 4 + (L + 1) * 4 + 8)
    ach = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "drafted blocks verified per second on 1 MI355X", "value": round(B / (ms * 1e-3), 1),
        "unit": "blocks/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + " verify", "blocks": B, "block": L, "vocab": V,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "dflash_verify_accept", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes": nbytes, "mean_launch_ms": round(ms, 5), "traffic": None},
        "cpu_baseline": None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="verify_t8")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
    ap.add_argument("--breakdown", action="store_true", help="per-kernel times on stderr")
    ap.add_argument("--router", action="store_true",
                    help="time moe_router_topk (router projection + top-k) instead of the layer")
    ap.add_argument("--verify", action="store_true",
                    help="time dflash_verify_accept on the workload's sequences (T / 8 blocks of 8)")
    ap.add_argument("--save-counts", default=None,
                    help="write the per-expert row counts of the workload to this .npy")
    ap.add_argument("--summarize", action="store_true",
                    help="summarise rocprofv3 output (no GPU): --stats-dir, --fetch-dir, "
                         "--write-dir, --counts, --command")
    ap.add_argument("--stats-dir", default=None)
    ap.add_argument("--fetch-dir", default=None)
    ap.add_argument("--write-dir", default=None)
    ap.add_argument("--counts", default=None)
    ap.add_argument("--command", default=None)
    args = ap.parse_args()

    if args.summarize:
        summarize_profiles(args)
        return

    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d is not supported "
              "(the layer is measured on one MI355X)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import mxfp4_moe_expert_route_amd as mm
    import workloads

    cfg = workloads.CONFIGS[args.config]
    if args.router:
        bench_router(args, cfg, torch, mm, workloads)
        return
    if args.verify:
        bench_verify(args, cfg, torch, mm, workloads)
        return
    steps = args.steps or (200 if cfg.T <= 512 else 30)
    warmup = args.warmup if args.warmup is not None else (20 if cfg.T <= 512 else 5)
    dev = torch.device("cuda:0")
    mm._lib.lib()

    t0 = time.perf_counter()
    whost = workloads.all_weights(cfg, 0)
    x_bits = workloads.gen_x_bits(cfg, 0)
    logits_h = workloads.gen_logits(cfg, x_bits, 0)
    log("inputs generated in %.1f s (%.2f GB of expert weights)"
        % (time.perf_counter() - t0, cfg.E * cfg.expert_bytes() / 1e9))
    names = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")
    w0 = {k: torch.from_numpy(whost[k]).to(dev) for k in names}
    w1 = {k: v.clone() for k, v in w0.items()}           # second copy for cache rotation
    wsets = (w0, w1)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(logits_h).to(dev)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    b = mm.LayerBuffers(T, H, I, E, k, dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        w = wsets[i & 1]
        mm.moe_route_permute(logits, k, b.topk_ids, b.topk_w, b.counts, b.offsets,
                             b.sorted_pairs, b.pair_to_row, b.workspace)
        if ev is not None:
            ev[0].record(stream)
        mm.moe_mxfp4_gate_up_swiglu(x, b.sorted_pairs, b.offsets, k, w["w13_codes"],
                                    w["w13_scales"], b.h)
        if ev is not None:
            ev[1].record(stream)
        mm.moe_mxfp4_down(b.h, b.offsets, k, w["w2_codes"], w["w2_scales"], b.y)
        mm.moe_combine(b.y, b.topk_w, b.pair_to_row, b.out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        step(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / steps
    gu_ms = float(np.mean([a.elapsed_time(bb) for a, bb in evs]))
    log("wall %.3f ms/step, events %.3f ms/step, gate_up %.3f ms"
        % (wall * 1e3 / steps, ms_step, gu_ms))

    counts = b.counts.cpu().numpy()
    if args.save_counts:
        np.save(args.save_counts, counts)
    touched = int((counts > 0).sum())
    w13_bytes = 2 * I * H // 2 + 2 * I * H // 32
    w2_bytes = H * I // 2 + H * I // 32
    layer_weight_bytes = touched * (w13_bytes + w2_bytes)
    gu_bytes = touched * w13_bytes + T * H * 2          # weights streamed + x read once
    flops = 6.0 * T * k * H * I
    eff_gbps = layer_weight_bytes / (ms_step * 1e-3) / 1e9
    gu_gbps = gu_bytes / (gu_ms * 1e-3) / 1e9
    tokens_per_s = T / (ms_step * 1e-3)

    if args.breakdown:
        names_k = ("route+permute", "gate_up", "down", "combine")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(20)]
        for r in range(20):
            w = wsets[r & 1]
            e = ev[r]
            e[0].record(stream)
            mm.moe_route_permute(logits, k, b.topk_ids, b.topk_w, b.counts, b.offsets,
                                 b.sorted_pairs, b.pair_to_row, b.workspace)
            e[1].record(stream)
            mm.moe_mxfp4_gate_up_swiglu(x, b.sorted_pairs, b.offsets, k, w["w13_codes"],
                                        w["w13_scales"], b.h)
            e[2].record(stream)
            mm.moe_mxfp4_down(b.h, b.offsets, k, w["w2_codes"], w["w2_scales"], b.y)
            e[3].record(stream)
            mm.moe_combine(b.y, b.topk_w, b.pair_to_row, b.out)
            e[4].record(stream)
        torch.cuda.synchronize()
        for i, n in enumerate(names_k):
            t = np.median([ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(20)])
            log("  %-8s %8.1f us" % (n, t * 1e3))

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(cfg, x_bits, logits_h, whost, args.cpu_budget)
        log("cpu baseline: %.3f tokens/s (%s)" % (cpu["value"], cpu["sample"]))

    traffic = measured_traffic("moe_mxfp4_gate_up_swiglu", cfg.name)
    # the gate/up contraction is bound by HBM when its flops per algorithmic
    # byte are below the machine balance (bf16 MFMA peak / HBM peak), else by
    # the matrix cores
    gu_flops = 4.0 * T * k * H * I
    if gu_flops / gu_bytes < BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roofline = {"kernel": "moe_mxfp4_gate_up_swiglu", "bound": "hbm",
                    "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(gu_gbps / HBM_PEAK_GBPS, 4)}
    else:
        tflops = gu_flops / (gu_ms * 1e-3) / 1e12
        roofline = {"kernel": "moe_mxfp4_gate_up_swiglu", "bound": "mfma",
                    "achieved": round(tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
    roofline.update({"traffic": traffic, "algorithmic_bytes": gu_bytes,
                     "algorithmic_flops": gu_flops, "mean_launch_ms": round(gu_ms, 5)})
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "top_k": k, "weight_format": "mxfp4 (E2M1, E8M0 per 32)",
                   "touched_experts": touched, "weight_bytes_touched": layer_weight_bytes,
                   "seed": 0, "parallelism": "none (1 GPU)"},
        "effective_weight_GBps": round(eff_gbps, 1),
        "hbm_frac_layer": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "mfma_frac_layer": round(flops / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
