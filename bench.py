"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

One step = the whole layer (moe_route_permute (top-k routing and grouping by
expert) -> moe_mxfp4_gate_up_swiglu -> moe_mxfp4_down -> moe_combine) over one
batch of synthetic tokens, inputs resident in HBM.  Default workload: the
page-shaped layer (hidden 6144, 384 experts, top-8, intermediate 2048, MXFP4
block 32) verifying one sequence's 8-token draft block.  Two copies of the
expert weights alternate between steps so the 256 MB last-level cache cannot
serve them.

Each workload runs --warmup steps, then more until --warm-seconds have passed
(the clocks settle under sustained load), then four timed passes of --steps
steps: the headline region (two events around all steps), per-step events
(median / p10 / p90), events around every entry point (per-kernel times) and
events around each contraction alone (the roofline's launch times).
The verify_t8 run also times the same step through the persistent decode
layer entry point (one kernel), then verify_t64, zipf_t512 and prefill_t8192
on the same weights with the same flags.

Prints ONE JSON line on stdout; diagnostics go to stderr.
  value         tokens/s of the whole layer (headline region)
  roofline      the gate/up contraction (the kernel that streams 2/3 of the
                weight bytes): algorithmic bytes per launch / its mean duration
                from HIP events just before and after its calls, against 8 TB/s
                (or the bf16 MFMA peak where it is compute-bound)
  workloads     the same figures for the other page-shaped workloads
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

import workloads  # noqa: E402  (seeded input generators; no layer arithmetic)

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
    "moe_mxfp4_decode_layer": ("k_decode_layer",),
}
# source files of each kernel family; every measurement also depends on the
# shared helpers and on the host code that picks the kernel
KERNEL_FILES = {"k_decode<": ("expert_decode.hip", "decode_stream.hpp"),
                "k_decode_layer": ("decode_layer.hip", "decode_stream.hpp", "routing.hpp"),
                "k_gate_up": ("expert_stream.hip",), "k_down": ("expert_stream.hip",),
                "k_dense": ("expert_dense.hip",)}
COMMON_FILES = ("common.hpp", "expert_stream.hip", "api.hip")


def kernel_sources(kernel_names):
    files = set(COMMON_FILES)
    for n in kernel_names:
        for k, fs in KERNEL_FILES.items():
            if k in n:
                files.update(fs)
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
    return {"moe_mxfp4_decode_layer": touched * (w13 + w2) + T * H * 2 + T * cfg.E * 4
            + T * H * 4,
            "moe_mxfp4_gate_up_swiglu": touched * w13 + T * H * 2,
            "moe_mxfp4_down": touched * w2, "touched": touched}


def _short_kernel_name(n):
    return n.replace("mxm::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _is_phase_marker(name):
    # torch.cuda._sleep, launched by time_layer at the start of each workload
    return "spin_kernel" in name or "sleep" in name.lower()


def trace_tables(trace_dir, phases, show=None):
    """Per-workload kernel statistics from a rocprofv3 kernel trace of one
    bench.py run: the dispatches are cut at the marker kernel that starts
    each workload, in the order `phases` names them."""
    rows = _csv_rows(_find_csv(trace_dir, "kernel_trace.csv"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    seg, per = -1, {}
    for r in rows:
        name = r["Kernel_Name"]
        if _is_phase_marker(name):
            seg += 1
            continue
        if seg < 0 or seg >= len(phases):
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(phases[seg], {}).setdefault(_short_kernel_name(name), []).append(dur)
    out = []
    for ph in phases:
        if show and ph not in show:
            continue
        ks = per.get(ph, {})
        tot = sum(sum(v) for v in ks.values()) or 1.0
        out += ["Workload %s (every dispatch of the workload: warm-up and timed passes):" % ph, "",
                "| kernel | calls | average (us) | median (us) | min (us) | max (us) | share |",
                "|---|---|---|---|---|---|---|"]
        for n, v in sorted(ks.items(), key=lambda kv: -sum(kv[1])):
            out.append("| %s | %d | %.1f | %.1f | %.1f | %.1f | %.1f%% |" % (
                n, len(v), np.mean(v), np.median(v), min(v), max(v), 100.0 * sum(v) / tot))
        out.append("")
    return out


def mfma_table(d, cfg, counts):
    """Matrix-core counters of the dense contractions from one rocprofv3 --pmc
    run: SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs), GRBM_GUI_ACTIVE
    (the dispatch's GPU cycles, summed over the XCDs) and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA work in units of 512 flops).
    Busy = busy cycles / (active cycles per XCD x SIMDs): the share of the
    kernel's own cycles the matrix units worked, at whatever clock it ran;
    clock = active cycles per XCD / the dispatch's duration."""
    agent = [r for r in _csv_rows(_find_csv(d, "agent_info.csv")) if int(r.get("Simd_Count") or 0) > 0]
    nxcc = int(agent[0]["Num_Xcc"]) if agent else 8
    nsimd = int(agent[0]["Simd_Count"]) if agent else 1024
    rows = _csv_rows(_find_csv(d, "counter_collection.csv"))
    per = {}
    for r in rows:
        n = _short_kernel_name(r["Kernel_Name"])
        if "k_dense" not in n:
            continue
        v = per.setdefault(n, {}).setdefault(r["Dispatch_Id"], {})
        v[r["Counter_Name"]] = float(r["Counter_Value"])
        v["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = ["Matrix-core counters (rocprofv3 --pmc, %d XCDs, %d SIMDs; per dispatch, averaged):"
           % (nxcc, nsimd), "",
           "| kernel | dispatches | MFMA busy share of the kernel's cycles | clock (GHz) | "
           "busy x clock / 2.4 GHz | bf16 MFMA flops (counter) | flops of all rows (4 or 2 T k H I) |",
           "|---|---|---|---|---|---|---|"]
    R = cfg.T * cfg.k
    for n, disp in sorted(per.items()):
        vs = [v for v in disp.values() if "SQ_VALU_MFMA_BUSY_CYCLES" in v and v.get("GRBM_GUI_ACTIVE")]
        busy = np.mean([v["SQ_VALU_MFMA_BUSY_CYCLES"] / (v["GRBM_GUI_ACTIVE"] / nxcc * nsimd)
                        for v in vs])
        clk = np.mean([v["GRBM_GUI_ACTIVE"] / nxcc / v["ns"] for v in vs])
        flops = np.mean([v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 for v in disp.values()
                         if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in v])
        alg = (4.0 if "true" in n else 2.0) * R * cfg.H * cfg.I
        out.append("| %s | %d | %.3f | %.2f | %.3f | %.4g | %.4g |"
                   % (n, len(disp), busy, clk, busy * clk / 2.4, flops, alg))
    out += ["", "The counted flops exceed those of the rows by the padding of each expert's last "
            "16-row token subtile.", ""]
    return out


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
    if args.trace_dir:
        out += trace_tables(args.trace_dir, (args.phases or cfg.name).split(","),
                            args.show.split(",") if args.show else None)
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
    if args.mfma_dir:
        out += mfma_table(args.mfma_dir, cfg, np.load(args.counts) if args.counts else None)
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
                if not by_kernel:
                    continue
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
                "bytes_per_launch": int(round(v["FETCH_SIZE"])) + int(round(v["WRITE_SIZE"])),
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


# ---------------------------------------------------------------------------
# the layer benchmark

# the other page-shaped workloads (same layer weights as verify_t8), timed in
# the same run after the headline workload
EXTRA_WORKLOADS = ("verify_t64", "zipf_t512", "prefill_t8192")


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


class ClockSampler:
    """Samples the GPU's current shader and memory clock levels from the
    driver's sysfs files (pp_dpm_sclk / pp_dpm_mclk, the level marked '*')
    in a host thread while the GPU runs; no GPU call, no child process."""

    def __init__(self, torch):
        self.paths = {}
        try:
            p = torch.cuda.get_device_properties(0)
            bus = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id,
                                         p.pci_device_id)
            base = "/sys/bus/pci/devices/%s" % bus
            for clk in ("sclk", "mclk", "fclk"):
                f = "%s/pp_dpm_%s" % (base, clk)
                if os.path.exists(f):
                    self.paths[clk] = f
            self.device = bus
        except Exception as e:                     # noqa: BLE001 (report, do not fail)
            self.device = "unknown (%s)" % e
        self.samples = {c: [] for c in self.paths}
        self._stop = None
        self._thread = None

    def _read(self):
        import re
        for clk, f in self.paths.items():
            try:
                with open(f) as fh:
                    for line in fh:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                self.samples[clk].append(int(m.group(1)))
            except OSError:
                pass

    def start(self):
        import threading
        if not self.paths:
            return
        self._stop = threading.Event()

        def run():
            while not self._stop.wait(0.02):
                self._read()
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self):
        if not self.paths:
            return {"source": "pp_dpm sysfs files not readable", "device": self.device}
        out = {"source": "sysfs pp_dpm_* current level, sampled every 20 ms while the "
                         "layer ran", "device": self.device}
        for clk, v in self.samples.items():
            if v:
                out[clk + "_mhz"] = {"median": int(np.median(v)), "min": int(min(v)),
                                     "max": int(max(v)), "samples": len(v)}
        return out


def upload_weights(cfg, torch, dev):
    """Two device copies of all expert weights (steps alternate between them
    so the 256 MB last-level cache cannot serve the touched experts)."""
    t0 = time.perf_counter()
    whost = workloads.all_weights(cfg, 0)
    log("weights generated in %.1f s (%.2f GB of expert weights)"
        % (time.perf_counter() - t0, cfg.E * cfg.expert_bytes() / 1e9))
    names = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")
    w0 = {k: torch.from_numpy(whost[k]).to(dev) for k in names}
    w1 = {k: v.clone() for k, v in w0.items()}
    return whost, (w0, w1)


class LayerRun:
    """One workload's inputs, buffers and step function (the whole layer:
    routing + grouping, gate/up, down, combine on the current stream)."""

    def __init__(self, cfg, wsets, torch, mm, dev):
        self.cfg, self.wsets, self.torch, self.mm = cfg, wsets, torch, mm
        self.x_bits = workloads.gen_x_bits(cfg, 0)
        self.logits_h = workloads.gen_logits(cfg, self.x_bits, 0)
        self.x = torch.from_numpy(self.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        self.logits = torch.from_numpy(self.logits_h).to(dev)
        self.b = mm.LayerBuffers(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev)
        self.stream = torch.cuda.current_stream()
        self.n = 0                                  # steps run (for the weight copy parity)

    def step(self, ev=None, at=(0, 1, 2, 3, 4)):
        """One layer step; ev[i] is recorded at point i (0: before routing, 1:
        before gate/up, 2: before down, 3: before combine, 4: after) for the
        points listed in `at`."""
        mm, b, k = self.mm, self.b, self.cfg.k
        w = self.wsets[self.n & 1]
        self.n += 1

        def mark(i):
            if ev is not None and i in at:
                ev[i].record(self.stream)
        mark(0)
        mm.moe_route_permute(self.logits, k, b.topk_ids, b.topk_w, b.counts, b.offsets,
                             b.sorted_pairs, b.pair_to_row, b.workspace)
        mark(1)
        mm.moe_mxfp4_gate_up_swiglu(self.x, b.sorted_pairs, b.offsets, k, w["w13_codes"],
                                    w["w13_scales"], b.h)
        mark(2)
        mm.moe_mxfp4_down(b.h, b.offsets, k, w["w2_codes"], w["w2_scales"], b.y)
        mark(3)
        mm.moe_combine(b.y, b.topk_w, b.pair_to_row, b.out)
        mark(4)


def time_layer(run, steps, warmup, warm_s, clocks=None):
    """Warm up, then four passes of `steps` steps each:
      1. the headline region: two events around all steps, nothing inside;
      2. per-step times: one event between consecutive steps;
      3. per-entry-point times: events around each call of every step;
      4. each contraction alone: events just before and after its call (fewer
         markers between the kernels, for the roofline's launch times).
    Warm-up is `warmup` steps and then more until `warm_s` seconds have passed
    (the clocks settle under sustained load)."""
    torch = run.torch
    Ev = lambda: torch.cuda.Event(enable_timing=True)       # noqa: E731
    torch.cuda._sleep(1000)      # marks the start of this workload in a kernel trace
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    if clocks is not None:
        clocks.start()
    t0 = time.perf_counter()
    nwarm, batch = warmup, 1
    while time.perf_counter() - t0 < warm_s:
        for _ in range(batch):
            run.step()
        nwarm += batch
        torch.cuda.synchronize()
        batch = min(2 * batch, 512)
    warm_elapsed = time.perf_counter() - t0

    s = run.stream
    e0, e1 = Ev(), Ev()
    wall0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        run.step()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / steps

    evs = [Ev() for _ in range(steps + 1)]
    evs[0].record(s)
    for i in range(steps):
        run.step()
        evs[i + 1].record(s)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])

    kev = [[Ev() for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        run.step(kev[i])
    torch.cuda.synchronize()
    if clocks is not None:
        clocks.stop()
    parts = ("route_permute", "gate_up", "down", "combine")
    per_kernel = {p: np.array([kev[i][j].elapsed_time(kev[i][j + 1]) for i in range(steps)])
                  for j, p in enumerate(parts)}
    alone = {}
    for j, p in ((1, "gate_up"), (2, "down")):
        aev = [[Ev() for _ in range(5)] for _ in range(steps)]
        for i in range(steps):
            run.step(aev[i], at=(j, j + 1))
        torch.cuda.synchronize()
        alone[p] = np.array([aev[i][j].elapsed_time(aev[i][j + 1]) for i in range(steps)])
    res = {"ms_per_step": ms_step, "wall_ms_per_step": wall * 1e3 / steps,
           "per_step": per_step, "per_kernel": per_kernel, "alone": alone,
           "warmup_steps": nwarm,
           "warmup_s": warm_elapsed}
    log("%s: events %.4f ms/step (wall %.4f), per-step median %.4f p10 %.4f p90 %.4f; "
        "warm-up %d steps in %.2f s" % (run.cfg.name, ms_step, res["wall_ms_per_step"],
                                       np.median(per_step), np.percentile(per_step, 10),
                                       np.percentile(per_step, 90), nwarm, warm_elapsed))
    log("  " + ", ".join("%s %.1f us" % (p, np.median(v) * 1e3) for p, v in per_kernel.items())
        + "; alone: " + ", ".join("%s %.1f us" % (p, np.mean(v) * 1e3) for p, v in alone.items()))
    return res


def time_decode_layer(run, steps, warmup, warm_s):
    """The same workload through moe_mxfp4_decode_layer (the whole layer as
    one persistent kernel), timed like time_layer's first two passes; None
    when that entry point does not take the sizes."""
    torch, mm, cfg, b = run.torch, run.mm, run.cfg, run.b
    ws = mm.decode_layer_workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, b.out.device)
    if ws is None:
        return None

    def step():
        w = run.wsets[run.n & 1]
        run.n += 1
        mm.moe_mxfp4_decode_layer(run.x, run.logits, cfg.k, w["w13_codes"], w["w13_scales"],
                                  w["w2_codes"], w["w2_scales"], ws, buffers=b)
    Ev = lambda: torch.cuda.Event(enable_timing=True)       # noqa: E731
    torch.cuda._sleep(1000)      # marks the start of this phase in a kernel trace
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, batch = time.perf_counter(), 1
    while time.perf_counter() - t0 < warm_s:
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        batch = min(2 * batch, 512)
    s = run.stream
    e0, e1 = Ev(), Ev()
    e0.record(s)
    for _ in range(steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    evs = [Ev() for _ in range(steps + 1)]
    evs[0].record(s)
    for i in range(steps):
        step()
        evs[i + 1].record(s)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    err = int(ws.view(torch.int32)[2].item())
    log("%s decode layer (one persistent kernel): %.4f ms/step, median %.4f, error word %d"
        % (cfg.name, ms, np.median(per), err))
    return {"entry": "moe_mxfp4_decode_layer", "ms_per_step": round(ms, 5),
            "ms_per_step_p10": round(float(np.percentile(per, 10)), 5),
            "ms_per_step_median": round(float(np.median(per)), 5),
            "ms_per_step_p90": round(float(np.percentile(per, 90)), 5),
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "error_word": err}


def layer_figures(cfg, counts, res):
    """Rates of one timed workload: tokens/s, effective weight bandwidth,
    fractions of the HBM and bf16 MFMA peaks, and the same for each
    contraction (mean of its per-call event times)."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    alg = _algorithmic_bytes(cfg, counts)
    touched = alg["touched"]
    w13 = 2 * I * H // 2 + 2 * I * H // 32
    w2 = H * I // 2 + H * I // 32
    layer_bytes = touched * (w13 + w2)
    ms = res["ms_per_step"]
    per_step = res["per_step"]
    eff = layer_bytes / (ms * 1e-3) / 1e9
    out = {"tokens": T, "touched_experts": touched, "weight_bytes_touched": layer_bytes,
           "ms_per_step": round(ms, 5),
           "ms_per_step_p10": round(float(np.percentile(per_step, 10)), 5),
           "ms_per_step_median": round(float(np.median(per_step)), 5),
           "ms_per_step_p90": round(float(np.percentile(per_step, 90)), 5),
           "tokens_per_s": round(T / (ms * 1e-3), 1),
           "effective_weight_GBps": round(eff, 1),
           "hbm_frac_layer": round(eff / HBM_PEAK_GBPS, 4),
           "mfma_frac_layer": round(6.0 * T * k * H * I / (ms * 1e-3) / 1e12 /
                                    BF16_MFMA_PEAK_TFLOPS, 4)}
    for entry, part, fl in (("moe_mxfp4_gate_up_swiglu", "gate_up", 4.0),
                            ("moe_mxfp4_down", "down", 2.0)):
        t = float(np.mean(res["alone"][part]))
        nbytes, flops = alg[entry], fl * T * k * H * I
        if flops / nbytes < BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
            ach = nbytes / (t * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                 "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4)}
        else:
            ach = flops / (t * 1e-3) / 1e12
            r = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4)}
        r.update({"kernel": entry, "algorithmic_bytes": int(nbytes), "algorithmic_flops": flops,
                  "mean_launch_ms": round(t, 5),
                  "median_launch_ms": round(float(np.median(res["alone"][part])), 5),
                  "traffic": measured_traffic(entry, cfg.name)})
        out[part] = r
    return out


def stream_probe(args, torch, mm):
    """Streaming-read ceiling: mxm_stream_xor over a buffer 16x the last-level
    cache, default cache policy and non-temporal loads."""
    dev = torch.device("cuda:0")
    nbytes = 16 * LLC_BYTES
    steps = args.steps or 20
    warmup = args.warmup if args.warmup is not None else 5
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    want = int(np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32)))
    res = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    out = {}
    for nt in (0, 1):
        for _ in range(warmup):
            mm.mxm_stream_xor(src, res, nt)
        torch.cuda.synchronize()
        res.zero_()
        torch.cuda.synchronize()
        mm.mxm_stream_xor(src, res, nt)
        torch.cuda.synchronize()
        ok = (int(res.item()) & 0xffffffff) == want
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(s)
        for i in range(steps):
            mm.mxm_stream_xor(src, res, nt)
            evs[i + 1].record(s)
        torch.cuda.synchronize()
        t = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
        gbps = nbytes / (np.median(t) * 1e-3) / 1e9
        out["nontemporal" if nt else "default"] = {
            "GBps_median": round(gbps, 1), "GBps_best": round(nbytes / (t.min() * 1e-3) / 1e9, 1),
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "ms_median": round(float(np.median(t)), 4),
            "xor_checked": ok}
        log("stream probe (%s): %.1f GB/s median, xor %s"
            % ("non-temporal" if nt else "default", gbps, "ok" if ok else "MISMATCH"))
    best = max(v["GBps_median"] for v in out.values())
    print(json.dumps({
        "metric": "streaming HBM read GB/s on 1 MI355X", "value": best, "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "stream_xor %d MiB" % (nbytes >> 20), "bytes": nbytes},
        "roofline": {"kernel": "mxm_stream_xor", "bound": "hbm", "achieved": best,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(best / HBM_PEAK_GBPS, 4),
                     "traffic": None},
        "policies": out, "cpu_baseline": None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="minimum warm-up time per workload, after the --warmup steps")
    ap.add_argument("--config", default="verify_t8")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --config (by default the verify_t8 run also times "
                         "verify_t64, zipf_t512 and prefill_t8192 on the same weights)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
    ap.add_argument("--router", action="store_true",
                    help="time moe_router_topk (router projection + top-k) instead of the layer")
    ap.add_argument("--verify", action="store_true",
                    help="time dflash_verify_accept on the workload's sequences (T / 8 blocks of 8)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="time the streaming-read probe (the HBM read ceiling) instead")
    ap.add_argument("--save-counts", default=None,
                    help="write the per-expert row counts of the workload to this .npy")
    ap.add_argument("--summarize", action="store_true",
                    help="summarise rocprofv3 output (no GPU): --stats-dir or --trace-dir, "
                         "--fetch-dir, --write-dir, --counts, --command")
    ap.add_argument("--stats-dir", default=None)
    ap.add_argument("--trace-dir", default=None)
    ap.add_argument("--phases", default=None,
                    help="with --trace-dir: comma-separated workload names, in run order")
    ap.add_argument("--show", default=None,
                    help="with --trace-dir: the phases to print (default: all)")
    ap.add_argument("--fetch-dir", default=None)
    ap.add_argument("--mfma-dir", default=None,
                    help="rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    ap.add_argument("--write-dir", default=None)
    ap.add_argument("--counts", default=None)
    ap.add_argument("--command", default=None)
    args = ap.parse_args()

    if args.summarize:
        summarize_profiles(args)
        return

    if args.gpus != 1:
        print("bench.py: the layer is measured on exactly one GPU; --gpus %d is not supported "
              "(one MI355X runs the whole layer; sharding is not implemented)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mxfp4_moe_expert_route_amd as mm

    cfg = workloads.CONFIGS[args.config]
    if args.router:
        bench_router(args, cfg, torch, mm, workloads)
        return
    if args.verify:
        bench_verify(args, cfg, torch, mm, workloads)
        return
    mm._lib.lib()
    if args.stream_probe:
        stream_probe(args, torch, mm)
        return
    steps = args.steps or (200 if cfg.T <= 512 else 30)
    warmup = args.warmup if args.warmup is not None else (20 if cfg.T <= 512 else 5)
    dev = torch.device("cuda:0")

    whost, wsets = upload_weights(cfg, torch, dev)
    clocks = ClockSampler(torch)
    run = LayerRun(cfg, wsets, torch, mm, dev)
    res = time_layer(run, steps, warmup, args.warm_seconds, clocks)
    counts = run.b.counts.cpu().numpy()
    if args.save_counts:
        np.save(args.save_counts, counts)
    fig = layer_figures(cfg, counts, res)
    fused = time_decode_layer(run, steps, warmup, args.warm_seconds)
    if fused is not None:
        fused["hbm_frac_layer"] = round(fig["weight_bytes_touched"] / (fused["ms_per_step"] * 1e-3)
                                        / 1e9 / HBM_PEAK_GBPS, 4)
        fused["vs_multi_launch"] = round(fig["ms_per_step"] / fused["ms_per_step"], 4)

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(cfg, run.x_bits, run.logits_h, whost, args.cpu_budget)
        log("cpu baseline: %.3f tokens/s (%s)" % (cpu["value"], cpu["sample"]))
    del whost

    extra = {}
    if not args.no_extra and cfg.name == "verify_t8":
        del run
        for name in EXTRA_WORKLOADS:
            c2 = workloads.CONFIGS[name]
            assert c2.lid == cfg.lid and (c2.H, c2.I, c2.E, c2.k) == (cfg.H, cfg.I, cfg.E, cfg.k)
            r2 = LayerRun(c2, wsets, torch, mm, dev)
            res2 = time_layer(r2, steps, warmup, args.warm_seconds)
            extra[name] = layer_figures(c2, r2.b.counts.cpu().numpy(), res2)
            del r2
            torch.cuda.empty_cache()

    roofline = dict(fig["gate_up"])
    line = {
        "metric": METRIC,
        "value": fig["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "top_k": cfg.k,
                   "weight_format": "mxfp4 (E2M1, E8M0 per 32)",
                   "touched_experts": fig["touched_experts"],
                   "weight_bytes_touched": fig["weight_bytes_touched"],
                   "seed": 0, "parallelism": "none (1 GPU)"},
        "effective_weight_GBps": fig["effective_weight_GBps"],
        "hbm_frac_layer": fig["hbm_frac_layer"],
        "mfma_frac_layer": fig["mfma_frac_layer"],
        "ms_per_step_p10": fig["ms_per_step_p10"],
        "ms_per_step_median": fig["ms_per_step_median"],
        "ms_per_step_p90": fig["ms_per_step_p90"],
        "warmup_steps_run": res["warmup_steps"],
        "warmup_s": round(res["warmup_s"], 2),
        "roofline": roofline,
        "down": fig["down"],
        "decode_layer": fused,
        "workloads": extra,
        "clocks": clocks.summary(),
        "host_cpu": host_cpu_model(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
