"""Benchmark of the MC-Sparse hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large]

A step is one pass of the whole hot path on one batch of synthetic input
already resident in HBM: the anchor step (PDDP grouping, dense attention with
LSE, exact selection = group mass + top-K, token-sparse attention, residual)
followed by one reuse step (token-sparse attention with the cached residual)
on drifted inputs.  W untimed warm-up steps, then K timed steps bracketed by
torch.cuda.synchronize(); every stage is also timed with HIP events on the
stream the library launches on (torch's current stream).

The headline metric is the token-sparse attention speedup over this library's
own dense attention at the same shape (reuse-step sparse kernel vs the dense
kernel without LSE; the anchor's dense pass with LSE is reported beside it),
with the sparse kernel's MFMA-roofline fraction at the density-scaled FLOP
count 4*B*H*N*K*D, and beside it vanilla block-sparse attention at the same
budget (mean-pooled block selection, same sparse kernel).  One JSON line is
printed.  --all-workloads measures every workload and density instead (one
line each, with the anchor-path cost and the 50-step schedule with an anchor
every 10 steps by formula), then runs every workload's step schedule on
drifted inputs (the long workload: 50 steps, an anchor every 10).
--diagnostics scores the token and block selections of every workload by
attention recall and relative L1 error of the output, on the GPU, and runs
k-means grouping with its alignment inflation (mcs_kmeans).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "token-sparse attn speedup vs own dense @20% density, N=75600; MFMA util %"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="large", choices=["tiny", "small", "large", "long", "asset3d"])
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=32768)
    ap.add_argument("--cpu-sample-groups", type=int, default=591)
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--offload-layers", type=int, default=0,
                    help="time reuse steps over this many layers with the anchor cache resident vs offloaded")
    ap.add_argument("--torch-sdpa", action="store_true",
                    help="also time torch's scaled_dot_product_attention (flash backend) on the dense shape")
    ap.add_argument("--all-workloads", action="store_true",
                    help="every workload and density (one JSON line each) instead of the headline one, "
                         "then every workload's step schedule, run")
    ap.add_argument("--diagnostics", action="store_true",
                    help="attention recall and output error of the token and block selections on the GPU, "
                         "every workload at densities 0.1 / 0.2 / 0.3")
    return ap.parse_args()


def log(args, *msg):
    if not args.quiet:
        print(*msg, file=sys.stderr, flush=True)


def cpu_baseline(args, w, x, K, scale):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    from token_sparse_attention_amd import synth
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = min(affinity, blas)        # the oracle's matrix products run on the BLAS threads
    q = synth.to_f64(x["q"][0, 0])
    k = synth.to_f64(x["k"][0, 0])
    v = synth.to_f64(x["v"][0, 0])
    rows = min(args.cpu_sample_rows, w.N)
    t0 = time.perf_counter()
    oracle.dense_attention(q[:rows], k, v, scale)
    t_dense = time.perf_counter() - t0
    G = -(-w.N // w.C)
    ng = min(args.cpu_sample_groups, G)
    perm = synth.random_perm(1, 1, w.N, seed=1)[0, 0]
    idx = synth.random_index_sets(1, 1, G, K, w.N, seed=2)[0, 0]
    sub = np.concatenate([perm[g * w.C:(g + 1) * w.C] for g in range(ng)])
    # the oracle evaluates whole heads; give it exactly the sampled groups
    t0 = time.perf_counter()
    oracle.sparse_attention(q[sub], k, v, np.arange(sub.size), idx[:ng], w.C, scale)
    t_sparse = time.perf_counter() - t0
    dense_per_row = t_dense / rows
    sparse_per_row = t_sparse / sub.size
    n_rows = w.B * w.H * w.N
    return {
        "value": round(dense_per_row / sparse_per_row, 3),
        "unit": "x (oracle dense time / oracle sparse time per query row)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"head 0: dense attention of {rows} query rows over all {w.N} keys; sparse attention of "
                  f"{ng} groups of {w.C} queries over K={K} gathered keys; fp64 numpy",
        "dense_s_extrapolated": round(dense_per_row * n_rows, 1),
        "sparse_s_extrapolated": round(sparse_per_row * n_rows, 1),
        "sparse_tflops": round(4.0 * sub.size * K * w.D / t_sparse / 1e12, 4),
        "dense_tflops": round(4.0 * rows * w.N * w.D / t_dense / 1e12, 4),
        "affinity_cpus": affinity,
        "blas_threads": blas,
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or platform.machine()


def measured_traffic(workload: str, kernel_prefix: str):
    """HBM bytes per launch of an attention kernel from the committed counter
    summary, if it still describes the current attention sources (else None)."""
    from token_sparse_attention_amd import pmc
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("attn_source_hash") != pmc.source_hash(pmc.ATTN_SOURCES):
        return None
    for name, v in d["kernels"].items():
        if name.startswith(kernel_prefix) and not name.endswith(pmc.BSA_SUFFIX):
            return v["traffic_bytes"]
    return None


def measured_util(workload: str, kernel_prefix: str):
    """Shader clock and MFMA-busy share of a kernel from the committed counter
    summary, if it still describes the current kernel sources (else None)."""
    from token_sparse_attention_amd import pmc
    path = os.path.join(ROOT, "profiles", f"pmc_util_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("attn_source_hash") != pmc.source_hash(pmc.ATTN_SOURCES):
        return None
    for name, v in d["kernels"].items():
        if name.startswith(kernel_prefix) and not name.endswith(pmc.BSA_SUFFIX):
            return v
    return None


def torch_sdpa_ms(q, k, v, reps: int):
    """Context for the dense baseline: torch's scaled_dot_product_attention on
    the same bf16 tensors, restricted to its flash backend (an unsupported case
    raises instead of falling back to the bf16 math path).  Returns the mean
    ms, or the error text."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            f = torch.nn.functional.scaled_dot_product_attention
            f(q, k, v)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            for i in range(reps):
                ev[i].record()
                f(q, k, v)
            ev[reps].record()
            torch.cuda.synchronize()
        return round(float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])), 4)
    except Exception as ex:  # no flash backend for this device or shape
        return f"unavailable: {str(ex)[:160]}"


def _mean_ms(fn, reps: int) -> float:
    import torch
    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record()
        fn()
    ev[reps].record()
    torch.cuda.synchronize()
    return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


def measure_bsa(q0, k0, v0, q1, k1, v1, res, C, K, scale, reps: int, dense_nolse_ms: float) -> dict:
    """Vanilla block-sparse attention at the same budget, the pages' efficiency
    reference: contiguous query blocks of C, the K/64 key blocks of best
    mean-pooled score (mcs_select_blocks), then the same sparse kernel over
    the kept blocks' tokens with the residual epilogue (mcs_sparse_attn_ex)."""
    import torch

    from token_sparse_attention_amd import binding
    B, H, N, D = q0.shape
    ident = torch.arange(N, dtype=torch.int32, device=q0.device).expand(B, H, N).contiguous()
    ws = torch.empty(max(int(binding._lib.mcs_select_blocks_workspace(binding.dims_of(q0))), 16),
                     dtype=torch.uint8, device=q0.device)
    holder = {}

    def select():
        holder["sel"] = binding.select_blocks(q0, k0, ident, C, K, scale, workspace=ws)

    select_ms = _mean_ms(select, reps)
    bidx, bcnt = holder["sel"]
    out = torch.empty_like(q1)
    sparse_ms = _mean_ms(lambda: binding.sparse_attn_ex(q1, k1, v1, ident, bidx, C, kv_count=bcnt, residual=res,
                                                        scale=scale, out=out), reps)
    keys = float(bcnt.double().mean().item())          # real keys per group (short last block)
    flops = 4.0 * B * H * N * keys * D
    return {"select_ms": round(select_ms, 4), "sparse_ms": round(sparse_ms, 4),
            "mean_keys_per_group": round(keys, 1),
            "tflops": round(flops / (sparse_ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(flops / (sparse_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "efficiency_vs_ideal": round(dense_nolse_ms * keys / N / sparse_ms, 4)}


def measure(args, workload: str, density, steps: int, warmup: int) -> dict:
    """One workload at one density: W warm-up and K timed steps; returns the
    result object (without the CPU baseline)."""
    import torch

    from token_sparse_attention_amd import accounting, binding, synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[workload]
    s = density if density is not None else w.densities[0]
    K = accounting.k_from_density(s, w.N)
    G = accounting.num_groups(w.N, w.C)
    scale = 1.0 / math.sqrt(w.D)

    t0 = time.time()
    x0 = synth.generate(workload)
    x1 = synth.drift(workload, x0, step=1)
    log(args, f"[bench] inputs {workload} generated in {time.time() - t0:.1f}s")

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q0, k0, v0 = (dev_bf16(x0[t]) for t in "qkv")
    q1, k1, v1 = (dev_bf16(x1[t]) for t in "qkv")
    shape = tuple(q0.shape)
    B, H, N, D = shape
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    kv_idx = torch.empty((B, H, G, K), dtype=torch.int32, device=dev)
    o_dense = torch.empty_like(q0)
    o_sp = torch.empty_like(q0)
    res = torch.empty_like(q0)
    o_reuse = torch.empty_like(q0)
    ws_group = torch.empty(max(binding.group_workspace_bytes(shape, w.C), 16), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(binding.select_workspace_bytes(shape, w.C, K, all_heads=True), dtype=torch.uint8,
                         device=dev)

    stages = ["group", "dense_lse", "select", "sparse_anchor", "residual", "sparse_reuse"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        binding.group(q0, w.C, out=perm, workspace=ws_group)
        mark(1)
        binding.dense_attn(q0, k0, v0, scale, want_lse=True, out=o_dense, lse=lse)
        mark(2)
        binding.select(q0, k0, lse, perm, w.C, K, scale, out=kv_idx, workspace=ws_sel)
        mark(3)
        binding.sparse_attn(q0, k0, v0, perm, kv_idx, w.C, scale=scale, out=o_sp)
        mark(4)
        binding.residual_update(o_dense, o_sp, out=res)
        mark(5)
        binding.sparse_attn(q1, k1, v1, perm, kv_idx, w.C, residual=res, scale=scale, out=o_reuse)
        mark(6)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(args, "[bench] warm-up done")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(args, f"[bench] {steps} timed steps in {wall:.3f}s")

    per_stage = {name: [] for name in stages}
    for ev in events:
        for j, name in enumerate(stages):
            per_stage[name].append(ev[j].elapsed_time(ev[j + 1]))
    ms = {name: float(np.mean(v)) for name, v in per_stage.items()}

    # the dense baseline without LSE, same shape (isolated launches)
    reps = max(3, steps)
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    o_tmp = torch.empty_like(q0)
    binding.dense_attn(q0, k0, v0, scale, out=o_tmp)
    for i in range(reps):
        e0[i].record()
        binding.dense_attn(q0, k0, v0, scale, out=o_tmp)
    e0[reps].record()
    torch.cuda.synchronize()
    dense_nolse_ms = float(np.mean([e0[i].elapsed_time(e0[i + 1]) for i in range(reps)]))
    speedup = dense_nolse_ms / ms["sparse_reuse"]
    torch_sdpa = torch_sdpa_ms(q0, k0, v0, reps) if args.torch_sdpa else None
    bsa = measure_bsa(q0, k0, v0, q1, k1, v1, res, w.C, K, scale, reps, dense_nolse_ms)

    sparse_flops = accounting.sparse_flops(B, H, N, K, D)
    dense_flops = accounting.dense_flops(B, H, N, D)
    t_sparse = ms["sparse_reuse"] * 1e-3
    achieved = sparse_flops / t_sparse / 1e12
    ms_per_step = wall / steps * 1e3

    out = {
        "metric": METRIC,
        "value": round(speedup, 4),
        "unit": "x (own dense attention ms, no LSE / token-sparse attention ms, same shape)",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{workload}: B={B} H={H} N={N} D={D} C={w.C} density={s} K={K} G={G}",
                   "B": B, "H": H, "N": N, "D": D, "C": w.C, "density": s, "K": K,
                   "step": "anchor (group, dense+lse, select, sparse, residual) + reuse (sparse + residual)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(workload, f"attn_kernel<{D}, {w.C // 32}, true, true"),
                     "kernel": "attn_kernel (sparse, residual epilogue)",
                     "per_launch_flops": sparse_flops, "avg_launch_ms": round(ms["sparse_reuse"], 4),
                     "algorithmic_bytes": accounting.sparse_compulsory_bytes(B, H, N, K, D, w.C),
                     "gathered_bytes": accounting.sparse_gather_bytes(B, H, N, K, D, w.C)},
        "roofline_dense": {"bound": "mfma", "achieved": round(dense_flops / (ms["dense_lse"] * 1e-3) / 1e12, 2),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(dense_flops / (ms["dense_lse"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "stage_ms": {k: round(v, 4) for k, v in ms.items()},
        "dense_nolse_ms": round(dense_nolse_ms, 4),
        "torch_sdpa_flash_ms": torch_sdpa,
        "speedup_vs_dense_with_lse": round(ms["dense_lse"] / ms["sparse_reuse"], 4),
        "ideal_speedup": round(N / K, 4),
        "efficiency_vs_ideal": round(speedup * K / N, 4),
        "dense_tflops": round(dense_flops / (ms["dense_lse"] * 1e-3) / 1e12, 2),
        "select_tflops": round(accounting.select_flops(B, H, N, D) / (ms["select"] * 1e-3) / 1e12, 2),
        "block_sparse": bsa,
    }
    util = measured_util(workload, f"attn_kernel<{D}, {w.C // 32}, true, true")
    if util is not None:
        # context from the committed counter profile (another run, same kernel
        # sources): the clock this kernel ran at there (GRBM_GUI_ACTIVE over
        # the dispatch time) and the bf16 MFMA peak at that clock
        peak_clk = PEAK_BF16_TFLOPS * util["clock_ghz"] / 2.4
        out["roofline"]["from_profile"] = {
            "source": f"profiles/pmc_util_{workload}.json (a separate rocprofv3 --pmc run)",
            "clock_ghz": round(util["clock_ghz"], 3),
            "peak_at_that_clock": round(peak_clk, 1),
            "frac_at_that_clock": round(achieved / peak_clk, 4),
            "mfma_busy": round(util["mfma_busy"], 4)}
    # anchor-path cost, and the schedule of the long-video setting: 50 steps
    # with an anchor every 10 (5 anchors, 45 reuse steps)
    t_anchor = sum(ms[k] for k in ("group", "dense_lse", "select", "sparse_anchor", "residual"))
    out["anchor_ms"] = round(t_anchor, 4)
    sched = (5 * t_anchor + 45 * ms["sparse_reuse"]) / 50
    out["schedule_50x10"] = {"mean_step_ms": round(sched, 4),
                             "speedup_vs_50_dense": round(dense_nolse_ms / sched, 4),
                             "anchor_overhead_vs_dense": round(5 * (t_anchor - dense_nolse_ms) / (50 * dense_nolse_ms), 4)}
    if not args.no_cpu_baseline:
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(args, w, x0, K, scale)
        log(args, f"[bench] cpu baseline in {time.time() - t0:.1f}s")
    del x0, x1
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_offload(args, workload: str, layers: int, steps: int) -> dict:
    """Reuse steps over `layers` attention layers whose anchor entries (perm,
    kv ids, residual) are resident in HBM or offloaded to pinned host memory
    with the next layer prefetched during the current layer's attention."""
    import torch

    from token_sparse_attention_amd import accounting, binding, synth
    from token_sparse_attention_amd.cache import AnchorCache

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[workload]
    s = w.densities[0]
    K = accounting.k_from_density(s, w.N)
    scale = 1.0 / math.sqrt(w.D)
    x0 = synth.generate(workload)

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (dev_bf16(x0[t]) for t in "qkv")
    st = binding.anchor_step(q, k, v, w.C, K, scale)
    out_buf = torch.empty_like(q)
    res = {}
    for offload in (False, True):
        cache = AnchorCache(layers, offload=offload)
        for l in range(layers):          # every layer holds a copy of the same entry
            cache.put(l, st["perm"], st["kv_idx"], st["residual"])
        torch.cuda.synchronize()

        def reuse_step():
            for l in range(layers):
                e = cache.get(l)
                binding.sparse_attn(q, k, v, e.perm, e.kv_idx, w.C, residual=e.residual, scale=scale, out=out_buf)

        reuse_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            reuse_step()
        torch.cuda.synchronize()
        res[offload] = (time.perf_counter() - t0) / (steps * layers) * 1e3
        del cache
    # the copy of one entry alone (host -> device, pinned)
    host = [t.cpu().pin_memory() for t in (st["perm"], st["kv_idx"], st["residual"])]
    dst = [torch.empty_like(t) for t in (st["perm"], st["kv_idx"], st["residual"])]
    nbytes = sum(t.numel() * t.element_size() for t in host)
    for d_, h_ in zip(dst, host):
        d_.copy_(h_, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        for d_, h_ in zip(dst, host):
            d_.copy_(h_, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    t_copy = e0.elapsed_time(e1) / steps
    t_res, t_off = res[False], res[True]
    hidden = (t_res + t_copy - t_off) / t_copy
    return {"mode": "anchor-cache offload", "workload": workload, "layers": layers, "density": s, "K": K,
            "entry_bytes": nbytes, "h2d_ms_per_entry": round(t_copy, 3),
            "h2d_gbps": round(nbytes / (t_copy * 1e-3) / 1e9, 1),
            "reuse_ms_per_layer_resident": round(t_res, 3), "reuse_ms_per_layer_offloaded": round(t_off, 3),
            "transfer_hidden_fraction": round(max(0.0, min(1.0, hidden)), 3),
            "flop_per_byte": round(accounting.sparse_flops(w.B, w.H, w.N, K, w.D) / nbytes, 1)}


ALL_CONFIGS = [("tiny", 0.25), ("small", 0.20), ("large", 0.20), ("long", 0.25), ("long", 0.15), ("asset3d", 0.15)]

# the configurations' step schedules: (steps, anchor steps); the others reuse
# the last anchor's groups, ids and residual on drifted inputs
SCHEDULES = {"tiny": (2, (0,)), "small": (5, (0,)), "large": (2, (0,)), "long": (50, (0, 10, 20, 30, 40)),
             "asset3d": (10, (0,))}


def measure_schedule(args, workload: str) -> dict:
    """Runs the workload's schedule (every density at once, on the same drifted
    inputs): anchor steps run the whole anchor path, the others one token-sparse
    launch with the cached residual.  Each step's GPU time is taken with HIP
    events; generating the next step's inputs on the host is not timed."""
    import torch

    from token_sparse_attention_amd import accounting, binding, synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[workload]
    nsteps, anchors = SCHEDULES[workload]
    scale = 1.0 / math.sqrt(w.D)
    Ks = [accounting.k_from_density(s, w.N) for s in w.densities]

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x = synth.generate(workload)
    q, k, v = (dev_bf16(x[t]) for t in "qkv")
    shape = tuple(q.shape)
    B, H, N, D = shape
    G = accounting.num_groups(N, w.C)
    perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o_dense = torch.empty_like(q)
    o_sp = torch.empty_like(q)
    o = torch.empty_like(q)
    ws_group = torch.empty(max(binding.group_workspace_bytes(shape, w.C), 16), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(binding.select_workspace_bytes(shape, w.C, max(Ks), all_heads=True), dtype=torch.uint8,
                         device=dev)
    state = [{"idx": torch.empty((B, H, G, K), dtype=torch.int32, device=dev), "res": torch.empty_like(q),
              "anchor_ms": [], "reuse_ms": []} for K in Ks]
    dense_ms = _mean_ms(lambda: binding.dense_attn(q, k, v, scale, out=o_dense), 3)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t_host = time.time()
    for t in range(nsteps):
        if t > 0:
            x = synth.drift(workload, x, step=t)
            for dst, name in ((q, "q"), (k, "k"), (v, "v")):
                dst.copy_(dev_bf16(x[name]))
        for K, stt in zip(Ks, state):
            ev[0].record()
            if t in anchors:
                binding.group(q, w.C, out=perm, workspace=ws_group)
                binding.dense_attn(q, k, v, scale, want_lse=True, out=o_dense, lse=lse)
                binding.select(q, k, lse, perm, w.C, K, scale, out=stt["idx"], workspace=ws_sel)
                binding.sparse_attn(q, k, v, perm, stt["idx"], w.C, scale=scale, out=o_sp)
                binding.residual_update(o_dense, o_sp, out=stt["res"])
            else:
                binding.sparse_attn(q, k, v, perm, stt["idx"], w.C, residual=stt["res"], scale=scale, out=o)
            ev[1].record()
            torch.cuda.synchronize()
            (stt["anchor_ms"] if t in anchors else stt["reuse_ms"]).append(ev[0].elapsed_time(ev[1]))
    log(args, f"[bench] {workload} schedule of {nsteps} steps in {time.time() - t_host:.1f}s")
    out = {"workload": workload, "steps": nsteps, "anchor_steps": list(anchors), "dense_nolse_ms": round(dense_ms, 4),
           "densities": {}}
    for s_, K, stt in zip(w.densities, Ks, state):
        total = sum(stt["anchor_ms"]) + sum(stt["reuse_ms"])
        out["densities"][str(s_)] = {
            "K": K,
            "anchor_ms_mean": round(float(np.mean(stt["anchor_ms"])), 4),
            "reuse_ms_mean": round(float(np.mean(stt["reuse_ms"])), 4) if stt["reuse_ms"] else None,
            "mean_step_ms": round(total / nsteps, 4),
            "speedup_vs_dense_steps": round(dense_ms * nsteps / total, 4),
            "anchor_overhead_vs_dense": round(sum(a - dense_ms for a in stt["anchor_ms"]) / (nsteps * dense_ms), 4)}
    del x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


DIAG_DENSITIES = (0.1, 0.2, 0.3)


def measure_diagnostics(args, workload: str) -> list:
    """Attention recall and relative L1 error of the output, on the GPU, for the
    library's own selection (PDDP groups, exact token selection) and for
    vanilla block-sparse attention (contiguous query blocks, mean-pooled key
    blocks) at densities 0.1 / 0.2 / 0.3 of one workload's anchor inputs.
    Every query of every head is scored.  Budgets K = 128*floor(s*N/128), at
    least 128."""
    import torch

    from token_sparse_attention_amd import accounting, binding, synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[workload]
    scale = 1.0 / math.sqrt(w.D)
    x = synth.generate(workload)
    q, k, v = (torch.from_numpy(x[t].view(np.int16)).view(torch.bfloat16).to(dev) for t in "qkv")
    del x
    B, H, N, D = q.shape
    perm = binding.group(q, w.C)
    ident = torch.arange(N, dtype=torch.int32, device=dev).expand(B, H, N).contiguous()
    od, lse = binding.dense_attn(q, k, v, scale, want_lse=True, out_dtype=torch.float32)
    rows = B * H * N

    def quality(o_s, lse_s):
        rec, l1, l1r = binding.query_quality(lse, lse_s, od, o_s)
        sums = binding.row_sums(torch.stack([rec.view(-1), l1.view(-1), l1r.view(-1)])).cpu().numpy()
        return {"recall": round(float(sums[0] / rows), 4), "rel_l1": round(float(sums[1] / sums[2]), 4)}

    out = []
    for s_ in DIAG_DENSITIES:
        K = max(128, accounting.k_from_density(s_, N))
        idx = binding.select(q, k, lse, perm, w.C, K, scale)
        o_s, lse_s = binding.sparse_attn_ex(q, k, v, perm, idx, w.C, scale=scale, want_lse=True,
                                            out_dtype=torch.float32)
        token = quality(o_s, lse_s)
        del idx
        bidx, bcnt = binding.select_blocks(q, k, ident, w.C, K, scale)
        o_b, lse_b = binding.sparse_attn_ex(q, k, v, ident, bidx, w.C, kv_count=bcnt, scale=scale, want_lse=True,
                                            out_dtype=torch.float32)
        blocks = quality(o_b, lse_b)
        del bidx, bcnt, o_s, o_b
        out.append({"mode": "selection diagnostics (GPU, all queries)", "workload": workload, "density": s_, "K": K,
                    "token_sparse_pddp": token, "block_sparse_contiguous": blocks})
        log(args, f"[bench] diagnostics {workload} s={s_}: {out[-1]}")
    out.append(measure_kmeans(args, workload, q, k))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_kmeans(args, workload: str, q, k, rounds: int = 20) -> dict:
    """k-means grouping of head 0 on the GPU (mcs_kmeans): ceil(N/C) query
    clusters and ceil(N/64) key clusters, Lloyd rounds from distinct seeded
    rows (the same rows the CPU diagnostics start from), and the alignment
    inflation of padding them to whole tiles."""
    import torch

    from token_sparse_attention_amd import binding, synth
    w = synth.WORKLOADS[workload]
    N = w.N
    G = -(-N // w.C)
    rng = np.random.default_rng(7000 + 100 * w.cfg_id + 0)
    qi, ki = rng.choice(N, G, replace=False), rng.choice(N, -(-N // 64), replace=False)
    res = {}
    for name, x, idx, tile in (("queries", q[0, 0], qi, w.C), ("keys", k[0, 0], ki, 64)):
        init = x[torch.from_numpy(idx).to(x.device)].float().contiguous()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, _, inertia, sizes = binding.kmeans(x.contiguous(), init, rounds)
        e1.record()
        torch.cuda.synchronize()
        sz = sizes.cpu().numpy()
        sz = sz[sz > 0]
        res[name] = {"clusters": int(idx.size), "empty": int(idx.size - sz.size), "min_size": int(sz.min()),
                     "max_size": int(sz.max()), "inflation": round(float((-(-sz // tile) * tile).sum() / sz.sum()), 4),
                     "final_inertia": round(float(inertia[-1].item()), 2), "ms": round(e0.elapsed_time(e1), 2)}
    out = {"mode": "k-means grouping (GPU, head 0)", "workload": workload, "rounds": rounds, **res,
           "inflation_blocks": round(res["queries"]["inflation"] * res["keys"]["inflation"], 4)}
    log(args, f"[bench] k-means {workload}: {out}")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): every stage of the path is "
              "independent per (batch, head), so several GPUs would each run their own heads with no "
              "exchange, and no multi-GPU figure is measured here", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.offload_layers > 0:
        print(json.dumps(measure_offload(args, args.workload, args.offload_layers, max(2, args.steps))), flush=True)
        return
    if args.diagnostics:
        for wl in ("tiny", "small", "large", "long", "asset3d"):
            for line in measure_diagnostics(args, wl):
                print(json.dumps(line), flush=True)
        return
    if args.all_workloads:
        # one JSON line per (workload, density), then the measured schedule of
        # every workload; no CPU baseline
        args.no_cpu_baseline = True
        for wl, dens in ALL_CONFIGS:
            out = measure(args, wl, dens, args.steps, args.warmup)
            print(json.dumps(out), flush=True)
        for wl in ("tiny", "small", "large", "long", "asset3d"):
            print(json.dumps({"mode": "measured schedule", **measure_schedule(args, wl)}), flush=True)
        return
    out = measure(args, args.workload, args.density, args.steps, args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
