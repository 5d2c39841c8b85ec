#!/usr/bin/env python3
"""Benchmark of the DiG token-mixer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C2] [--gpus 1]

One step = one pass of the whole path over one batch of synthetic input:
gla_fwd (chunk-wise GLA forward in the step's scan direction, directions
cycled step by step) followed by srem_dwconv (3x3 depthwise conv in the scan
frame, stored back to canonical order = the direction remap); the full
2048^2 step (--config C4) also runs the adaLN modulation first.  Inputs are
resident in HBM before timing starts; input sets rotate so that consecutive
steps do not find their inputs in the 256 MB Infinity Cache.

Prints ONE JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (gla_fwd, HBM-bound) measured with HIP events on the stream
it runs on, and the fp64 CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "GLA fwd tokens/sec + % MFMA/HBM roofline, DiG-XL/2 shape T=4096 d=72"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gla_alg_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one gla_fwd call: read q, k, v, log_alpha, write o (bf16) + fp32 final state."""
    el = 2 if cfg.dtype == "bf16" else 4
    return cfg.B * cfg.H * cfg.T * cfg.d * el * 5 + cfg.B * cfg.H * cfg.d * cfg.d * 4


def gla_alg_flops(cfg, M=64) -> int:
    """Chunk-wise algorithmic flops: B*H*T*(4*M*d + 4*d^2) (QK^T, PV, Q~S, K^T V tiles)."""
    return cfg.B * cfg.H * cfg.T * (4 * M * cfg.d + 4 * cfg.d * cfg.d)


def bwd_alg_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one gla_bwd call: read q, k, v, log_alpha, do (bf16), write dq, dk,
    dv (bf16) and dlog_alpha (fp32).  The chunk states the implementation keeps in its workspace
    are not counted."""
    return cfg.B * cfg.H * cfg.T * cfg.d * (5 * 2 + 3 * 2 + 4)


def bwd_alg_flops(cfg, M=64) -> int:
    """Chunk-form algorithmic flops per token and head: the two M x M products (dO V^T, Q~K~^T),
    the three token-contracting products (A K~, A^T Q~, P^T dO) and the state terms (dO S^T,
    V D^T, K^ D, K^^T V, and the two scans' X^T Y): 2 * (2 M d + 3 M d + 6 d^2)."""
    return cfg.B * cfg.H * cfg.T * 2 * (5 * M * cfg.d + 6 * cfg.d * cfg.d)


def conv_alg_bytes(cfg) -> int:
    el = 2 if cfg.dtype == "bf16" else 4
    return 2 * cfg.B * cfg.T * cfg.C * el + cfg.C * 9 * 4


def traffic_record(cfg_key: str, kind: str = "fwd"):
    """Measured HBM bytes per gla_fwd launch (kind "fwd") or per gla_bwd call (kind "bwd": both
    kernels) from a committed rocprofv3 PMC summary, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", f"gla_{kind}_{cfg_key.lower()}_traffic.json")
    src = os.path.join(ROOT, "gated_linear_attention_gla_amd", "csrc",
                       "gla_bwd.hip" if kind == "bwd" else "gla_bf16.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("kernel_src_sha256") != sha:
            return None
        return float(rec["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(cfg, x_cpu, budget_s: float = 20.0):
    """The fp64 oracle (as it stands) on this host: GLA + conv over a bounded sample of (b, h)
    units of the same workload, scaled to tokens/s of the whole batch."""
    import numpy as np
    from oracle import oracle

    threads = len(os.sched_getaffinity(0))
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    direction = cfg.direction(0)
    grid = (cfg.gh, cfg.gw)

    def run(sample):
        t0 = time.perf_counter()
        bs = sorted({b for b, _ in sample})
        for b in bs:
            hs = [h for bb, h in sample if bb == b]
            sl = lambda t: t[b:b + 1][:, :, hs].contiguous()
            if cfg.adaln:
                m = oracle.adaln_modulate(x_cpu["x_qkv"][:, b:b + 1], x_cpu["ada_scale"], x_cpu["ada_shift"],
                                          1e-6, x_cpu["ada_out_scale"], nthreads=threads)
                m = m.reshape(3, 1, cfg.T, cfg.H, cfg.d)[:, :, :, hs]
                q, k, v = (np.ascontiguousarray(m[i]) for i in range(3))
            else:
                q, k, v = sl(x_cpu["q"]), sl(x_cpu["k"]), sl(x_cpu["v"])
            o, _ = oracle.gla_fwd(q, k, v, sl(x_cpu["log_alpha"]), grid, direction, nthreads=threads)
            ch = np.concatenate([np.arange(h * cfg.d, (h + 1) * cfg.d) for h in hs])
            oracle.srem_dwconv(o.reshape(1, cfg.T, len(hs) * cfg.d), x_cpu["w"][ch], grid, direction,
                               nthreads=threads)
        return time.perf_counter() - t0

    # probe with as many units as threads, then size the sample to the budget
    probe = units[:min(len(units), threads)]
    tp = run(probe)
    n = len(probe)
    if tp < budget_s / 4 and n < len(units):
        want = int(n * (budget_s * 0.6) / max(tp, 1e-3) / threads) * threads
        want = max(n, min(len(units), want))
        if want > n:
            sample = units[:want]
            tp = run(sample)
            n = want
    est_full = tp * len(units) / n
    return {
        "value": cfg.B * cfg.T / est_full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {len(units)} (batch, head) units of {cfg.key} "
                  f"({'adaLN + ' if cfg.adaln else ''}GLA fwd + conv, dir {direction}, fp64, "
                  f"{threads} OpenMP threads): {tp:.2f} s, scaled to the whole batch",
    }


def cpu_baseline_bwd(cfg, x_cpu, do_cpu, budget_s: float = 20.0, order=None):
    """The fp64 oracle's backward on a bounded sample of (b, h) units, scaled to tokens/s of the
    whole batch."""
    from oracle import oracle

    threads = len(os.sched_getaffinity(0))
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    direction = cfg.direction(0)
    grid = (cfg.gh, cfg.gw)

    def run(sample):
        t0 = time.perf_counter()
        for b in sorted({b for b, _ in sample}):
            hs = [h for bb, h in sample if bb == b]
            sl = lambda t: t[b:b + 1][:, :, hs].contiguous()
            oracle.gla_bwd(sl(x_cpu["q"]), sl(x_cpu["k"]), sl(x_cpu["v"]), sl(x_cpu["log_alpha"]), grid,
                           direction, sl(do_cpu), nthreads=threads, order=order)
        return time.perf_counter() - t0

    probe = units[:min(len(units), threads)]
    tp = run(probe)
    n = len(probe)
    if tp < budget_s / 4 and n < len(units):
        want = int(n * (budget_s * 0.6) / max(tp, 1e-3) / threads) * threads
        want = max(n, min(len(units), want))
        if want > n:
            tp = run(units[:want])
            n = want
    est_full = tp * len(units) / n
    return {"value": cfg.B * cfg.T / est_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {len(units)} (batch, head) units of {cfg.key} (GLA backward, "
                      + ("zigzag order S_0" if order is not None else f"dir {direction}")
                      + f", fp64, {threads} OpenMP threads): {tp:.2f} s, scaled to the whole batch"}


def zigzag_tables(cfg, dev):
    """ZigMa's eight zigzag scan orders of the workload's grid as device tables."""
    from gated_linear_attention_gla_amd import scan_orders
    return [scan_orders.to_device(scan_orders.zigzag(j, cfg.gh, cfg.gw), dev) for j in range(8)]


def bench_fwd_ordered(a, dg, gen, torch) -> int:
    """gla_fwd over table scan orders (ZigMa's zigzag S_0..S_7, cycled): one step = one
    gla_fwd_ordered launch over rotating input sets, HIP events on the launch stream.  (The SREM
    conv is defined in the frame of the four grid orders, so it is not part of this step.)"""
    import numpy as np
    from oracle import oracle

    dev = torch.device("cuda:0")
    cfg = gen.CONFIGS[a.config]
    if cfg.adaln:
        print("bench.py --order zigzag: runs the GLA-only workloads (C1, C2, C3)", file=sys.stderr)
        return 2
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.d
    chunk = a.chunk or cfg.chunk
    nsets = a.sets or max(2, math.ceil(512e6 / gla_alg_bytes(cfg)))
    log(f"[bench] gla_fwd zigzag {cfg.key} {cfg.name}: B={B} H={H} T={T} ({cfg.gh}x{cfg.gw}) d={d}; {nsets} sets")
    sets = [gen.make_inputs(cfg.key, set_index=i, device=dev) for i in range(nsets)]
    o = torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    ws = dg.get_workspace(dev, dg.workspace_bytes(dg.DIG_BF16, B, T, H, d, d, chunk))
    tables = zigzag_tables(cfg, dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        x = sets[i % nsets]
        dg.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None, chunk=chunk, out=o, s_final=sf,
                   workspace=ws, order=tables[i % 8])

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(a.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(a.warmup + i)
        e1.record(stream)
        evs.append((e0, e1))
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / a.steps
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    avg = sum(ms) / len(ms)
    abytes, aflops = gla_alg_bytes(cfg), gla_alg_flops(cfg, chunk)
    achieved = abytes / (avg * 1e-3) / 1e9
    log(f"[bench] gla_fwd zigzag avg {avg * 1e3:.1f} us (median {ms[len(ms) // 2] * 1e3:.1f}), "
        f"{achieved:.0f} GB/s alg")
    cpu = None
    if not a.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        x0 = {k_: v_.cpu() for k_, v_ in sets[0].items() if isinstance(v_, torch.Tensor)}
        order0 = tables[0].cpu().numpy().astype(np.int64)
        t0 = time.perf_counter()
        oracle.gla_fwd(x0["q"], x0["k"], x0["v"], x0["log_alpha"], None, None, nthreads=threads, order=order0)
        tc = time.perf_counter() - t0
        cpu = {"value": B * T / tc, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"all {B * H} (batch, head) units of {cfg.key} (GLA fwd, zigzag order S_0, fp64, "
                         f"{threads} OpenMP threads): {tc:.2f} s"}
        log(f"[bench] cpu oracle: {cpu['value']:.3e} tokens/s on {threads} cores")
    rec = {
        "metric": "GLA fwd tokens/sec over zigzag scan orders, DiG-XL/2 shape T=4096 d=72",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations of the DiG latent-grid shape)",
        "config": {"workload": f"{cfg.key} {cfg.name}: GLA forward over ZigMa's zigzag scans S_0..S_7 "
                               f"(order tables, chunk {chunk})",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": d, "grid": [cfg.gh, cfg.gw],
                   "directions": ["zigzag S_0..S_7"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "gla_fwd_bf16_kernel (order table)",
                     "alg_bytes_per_launch": abytes, "avg_launch_us": avg * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def block_alg_flops(B, T, C, H, M=64) -> int:
    """Dense products of one block per token: q/k/v/gate (C -> 4C), out (C -> C), FFN (C -> 4C -> C):
    2 C^2 (4 + 1 + 8); plus the GLA's chunk-wise flops (4 M d + 4 d^2 per head and token)."""
    d = C // H
    return B * T * (2 * C * C * 13 + H * (4 * M * d + 4 * d * d))


def bench_block(a, dg, gen, torch) -> int:
    """One DiG-XL/2 block forward (dig_block_fwd) at the C2 latent grid (B=8, 64x64 tokens, C=1152,
    16 heads) on seeded synthetic weights: one step = one block call, directions cycled.  The MFMA
    roofline is taken on the block's largest product (tokens x 4C x C, the q/k/v/gate projection and
    the FFN's first layer), timed through dig_linear with HIP events on the same stream."""
    import numpy as np
    from oracle import oracle

    dev = torch.device("cuda:0")
    cfg = gen.CONFIGS["C2"]
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.d
    C = H * d
    grid = (cfg.gh, cfg.gw)
    log(f"[bench] DiG block C2 shape: B={B} T={T} ({cfg.gh}x{cfg.gw}) C={C} H={H}")
    x = gen.block_inputs(B, T, C, seed=cfg.seed, device=dev)
    w = {n: x[n] for n in dg.BLOCK_WEIGHTS}
    y = torch.empty_like(x["x"])
    n = dg.lib().dig_block_workspace_size(B, T, C, H)
    ws = dg.get_workspace(dev, int(n), key="block")
    stream = torch.cuda.current_stream(dev)

    def step(i):
        dg.block_fwd(x["x"], x["c"], w, grid, cfg.direction(i), H, out=y, workspace=ws)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(a.steps):
        step(a.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / a.steps
    aflops = block_alg_flops(B, T, C, H)
    # the largest product on its own, same operand sizes as inside the block
    xa = torch.randn(B * T, C, device=dev).to(torch.bfloat16)
    wa = (torch.randn(4 * C, C, device=dev) / math.sqrt(C)).to(torch.bfloat16)
    ya = torch.empty(B * T, 4 * C, dtype=torch.bfloat16, device=dev)
    for _ in range(5):
        dg.linear(xa, wa, out=ya)
    torch.cuda.synchronize()
    evs = []
    for _ in range(a.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dg.linear(xa, wa, out=ya)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    g_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
    g_flops = 2 * B * T * 4 * C * C
    g_tflops = g_flops / (g_ms * 1e-3) / 1e12
    log(f"[bench] block {ms_step * 1e3:.1f} us, {aflops / (ms_step * 1e-3) / 1e12:.0f} TFLOP/s alg; "
        f"largest product {g_ms * 1e3:.1f} us = {g_tflops:.0f} TFLOP/s")
    cpu = None
    if not a.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        xc = {k_: v_[:1].cpu() if k_ in ("x", "c") else v_.cpu() for k_, v_ in x.items()}
        tc0 = time.perf_counter()
        oracle.block_fwd(xc["x"], xc["c"], {n_: xc[n_] for n_ in dg.BLOCK_WEIGHTS}, grid, "l2r", H=H,
                         nthreads=threads)
        tc = time.perf_counter() - tc0
        cpu = {"value": T / tc, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"batch element 0 of 8 (T={T}, C={C}, fp64 numpy products + the C GLA and conv "
                         f"oracles, {threads} threads): {tc:.2f} s"}
        log(f"[bench] cpu oracle block: {cpu['value']:.3e} tokens/s on {threads} cores")
    rec = {
        "metric": "DiG block forward tokens/sec (adaLN-Zero, projections, GLA, FFN, SREM conv), DiG-XL/2 at 1024px",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations, conditioning and weights of the DiG-XL/2 block shape)",
        "config": {"workload": f"DiG-XL/2 block forward at the C2 latent grid (B={B}, {cfg.gh}x{cfg.gw} tokens, "
                               f"C={C}, {H} heads)",
                   "global_batch": B, "seq_len": T, "hidden": C, "heads": H, "grid": list(grid),
                   "directions": list(cfg.dirs), "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": g_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": g_tflops / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": f"gemm_bf16_kernel: largest product of the block ({B * T} x {4 * C} x {C}, bf16)",
                     "alg_flops_per_launch": g_flops, "avg_launch_us": g_ms * 1e3},
        "block": {"tflops_alg": aflops / (ms_step * 1e-3) / 1e12, "alg_flops_per_step": aflops},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_bwd(a, dg, gen, torch) -> int:
    """gla_bwd on the workload's shape: one step = one backward call (two launches on one
    stream: the forward state scan and the reverse state-gradient scan side by side, then the
    chunk gradients) over rotating input sets, timed with HIP events on that stream."""
    dev = torch.device("cuda:0")
    cfg = gen.CONFIGS[a.config]
    if cfg.adaln:
        print("bench.py --bwd: the backward bench runs the GLA-only workloads (C1, C2, C3)", file=sys.stderr)
        return 2
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.d
    grid = (cfg.gh, cfg.gw)
    chunk = a.chunk or cfg.chunk
    per_set = B * T * H * d * 2 * 5
    nsets = a.sets or max(2, math.ceil(512e6 / per_set))
    log(f"[bench] gla_bwd {cfg.key} {cfg.name}: B={B} H={H} T={T} ({cfg.gh}x{cfg.gw}) d={d}; {nsets} input sets")
    gen_do = torch.Generator(device=dev)
    sets = []
    for i in range(nsets):
        x = gen.make_inputs(cfg.key, set_index=i, device=dev)
        gen_do.manual_seed(cfg.seed + 4409 * (i + 1))
        do = torch.randn(B, T, H, d, generator=gen_do, device=dev).to(torch.bfloat16)
        sets.append((x, do))
    nbytes = dg.lib().gla_bwd_workspace_size(dg.DIG_BF16, B, T, H, d, d, chunk)
    ws = dg.get_workspace(dev, nbytes, key="bwd")
    stream = torch.cuda.current_stream(dev)
    tables = zigzag_tables(cfg, dev) if a.order == "zigzag" else None

    def step(i):
        x, do = sets[i % nsets]
        dg.gla_bwd(x["q"], x["k"], x["v"], x["log_alpha"], grid, cfg.direction(i), do, chunk=chunk,
                   need_ds0=False, workspace=ws, order=None if tables is None else tables[i % 8])

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(a.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(a.warmup + i)
        e1.record(stream)
        evs.append((e0, e1))
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / a.steps
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    avg = sum(ms) / len(ms)
    abytes, aflops = bwd_alg_bytes(cfg), bwd_alg_flops(cfg, chunk)
    achieved = abytes / (avg * 1e-3) / 1e9
    log(f"[bench] gla_bwd avg {avg * 1e3:.1f} us (median {ms[len(ms) // 2] * 1e3:.1f}), {achieved:.0f} GB/s alg, "
        f"{aflops / (avg * 1e-3) / 1e12:.1f} TFLOP/s alg")
    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle backward on a bounded sample ...")
        x0, do0 = sets[0]
        x_cpu = {k_: v_.cpu() for k_, v_ in x0.items() if isinstance(v_, torch.Tensor)}
        cpu = cpu_baseline_bwd(cfg, x_cpu, do0.cpu(), order=None if tables is None else tables[0].cpu().numpy())
        log(f"[bench] cpu oracle bwd: {cpu['value']:.3e} tokens/s on {cpu['cores']} cores")
    zz = tables is not None
    rec = {
        "metric": "GLA bwd tokens/sec (training backward" + (", zigzag scan orders" if zz else "")
                  + "), DiG-XL/2 shape T=4096 d=72",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations and output gradients of the DiG latent-grid shape)",
        "config": {"workload": f"{cfg.key} {cfg.name}: GLA backward (chunk {chunk}; dq, dk, dv, dlog_alpha)"
                               + (" over ZigMa's zigzag scans S_0..S_7 (order tables)" if zz else ""),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": d, "grid": list(grid),
                   "directions": ["zigzag S_0..S_7"] if zz else list(cfg.dirs), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None if zz else traffic_record(cfg.key, "bwd"),
                     "kernel": "gla_bwd (gla_bwd_scan, both directions in one launch, + gla_bwd_chunk)", "alg_bytes_per_launch": abytes,
                     "avg_launch_us": avg * 1e3},
        "gla_bwd": {"tflops_alg": aflops / (avg * 1e-3) / 1e12,
                    "mfma_frac": aflops / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    "median_us": ms[len(ms) // 2] * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


COPY_PROBE_BYTES = 256 << 20   # the plain copy whose counters calibrate FETCH_SIZE / WRITE_SIZE


def product_probe() -> int:
    """Launch sequence for PMC passes over the DiG block's largest product: five dig_linear calls
    of [B*T, C] x [4C, C]^T at the DiG-XL/2 block shape (B=8, 64x64 tokens, C=1152) on seeded
    operands."""
    import torch

    from gated_linear_attention_gla_amd import binding as dg

    dev = torch.device("cuda:0")
    B, T, C = 8, 64 * 64, 1152
    g = torch.Generator(device="cpu").manual_seed(0)
    x = (torch.randn(B * T, C, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    w = (torch.randn(4 * C, C, generator=g) / math.sqrt(C)).to(torch.bfloat16).to(dev)
    y = torch.empty(B * T, 4 * C, dtype=torch.bfloat16, device=dev)
    for _ in range(5):
        dg.linear(x, w, out=y)
    torch.cuda.synchronize()
    log("[bench] product probe: 5 x dig_linear 32768 x 4608 x 1152")
    return 0


def traffic_probe(cfg_key: str, chunk: int, bwd: bool = False) -> int:
    """Launch sequence for the two rocprofv3 PMC passes: three plain device copies of
    COPY_PROBE_BYTES (read + write of known size), then three gla_fwd launches of the workload
    (with bwd: three gla_bwd calls)."""
    import torch

    from gated_linear_attention_gla_amd import binding as dg
    from gated_linear_attention_gla_amd import inputs as gen

    dev = torch.device("cuda:0")
    cfg = gen.CONFIGS[cfg_key]
    src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    x = gen.make_inputs(cfg.key, set_index=0, device=dev)
    if cfg.adaln:
        m = dg.adaln_modulate(x["x_qkv"], x["ada_scale"], x["ada_shift"], 1e-6, x["ada_out_scale"])
        q, k, v = (m[j].view(cfg.B, cfg.T, cfg.H, cfg.d) for j in range(3))
    else:
        q, k, v = x["q"], x["k"], x["v"]
    # the same copy over 144-byte rows at the GLA's head stride: q [B, T, H, d]
    # rearranged to [B, H, T, d] by torch's strided copy kernel (reads and
    # writes q's bytes once each), a check that the copy's counter scaling
    # holds for rows of this size and stride
    qt = torch.empty(cfg.B, cfg.H, cfg.T, cfg.d, dtype=q.dtype, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    for _ in range(3):
        qt.copy_(q.permute(0, 2, 1, 3))
    if bwd:
        gen_do = torch.Generator(device=dev)
        gen_do.manual_seed(cfg.seed + 4409)
        do = torch.randn(cfg.B, cfg.T, cfg.H, cfg.d, generator=gen_do, device=dev).to(torch.bfloat16)
    torch.cuda.synchronize()
    for i in range(3):
        if bwd:
            dg.gla_bwd(q, k, v, x["log_alpha"], (cfg.gh, cfg.gw), cfg.direction(i), do, chunk=chunk or cfg.chunk,
                       need_ds0=False)
        else:
            dg.gla_fwd(q, k, v, x["log_alpha"], (cfg.gh, cfg.gw), cfg.direction(i), chunk=chunk)
    torch.cuda.synchronize()
    log(f"[bench] traffic probe done: {cfg.key}, 3 copies of {COPY_PROBE_BYTES} B, 3 gla_{'bwd' if bwd else 'fwd'} calls")
    return 0


def write_traffic(cfg_key: str, fetch_dir: str, write_dir: str, command: str, bwd: bool = False) -> int:
    """Turn the counter CSVs of the two PMC passes over --traffic-probe into the per-launch HBM
    traffic record read by traffic_record().  Each counter is scaled by bytes / counter of the copy.
    With bwd, a call's traffic is the sum of its two kernels' (medians over the three calls)."""
    import csv
    import glob
    import statistics

    from gated_linear_attention_gla_amd import inputs as gen

    cfg = gen.CONFIGS[cfg_key]

    def per_dispatch(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        names = ("gla_bwd_scan", "gla_bwd_chunk") if bwd else ("gla_fwd_bf16_kernel",)
        per = [[float(r["Counter_Value"]) * 1024 for r in rows if n in r["Kernel_Name"]] for n in names]
        # torch's same-dtype device copy is the runtime's blit kernel
        cp = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]]
        # torch's strided copy of q into [B, H, T, d] (elementwise kernel)
        st = [float(r["Counter_Value"]) * 1024 for r in rows if "direct_copy" in r["Kernel_Name"]]
        if min(len(g) for g in per) < 1 or len(cp) < 1:
            raise SystemExit(f"write_traffic: no gla/copy dispatches with {counter} under {d}")
        return (sum(statistics.median(g) for g in per), statistics.median(cp), len(per[-1]), len(cp),
                statistics.median(st) if st else None)

    gf, cf, ng, nc, sf_ = per_dispatch(fetch_dir, "FETCH_SIZE")
    gw, cw, _, _, sw_ = per_dispatch(write_dir, "WRITE_SIZE")
    kf, kw = COPY_PROBE_BYTES / cf, COPY_PROBE_BYTES / cw
    total = gf * kf + gw * kw
    q_bytes = cfg.B * cfg.T * cfg.H * cfg.d * 2
    strided = None if sf_ is None or sw_ is None else {
        "bytes": q_bytes, "fetch_raw": sf_, "write_raw": sw_, "fetch_scaled_over_bytes": sf_ * kf / q_bytes,
        "write_scaled_over_bytes": sw_ * kw / q_bytes}
    kind = "bwd" if bwd else "fwd"
    src = os.path.join(ROOT, "gated_linear_attention_gla_amd", "csrc", "gla_bwd.hip" if bwd else "gla_bf16.hip")
    alg = bwd_alg_bytes(cfg) if bwd else gla_alg_bytes(cfg)
    rec = {"kernel": "gla_bwd_scan + gla_bwd_chunk" if bwd else "gla_fwd_bf16_kernel", "workload": cfg_key,
           "kernel_src_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "bytes_per_launch": total, "fetch_bytes_raw": gf, "write_bytes_raw": gw,
           "copy_scale_fetch": kf, "copy_scale_write": kw, "copy_bytes": COPY_PROBE_BYTES,
           "alg_bytes_per_launch": alg, "gla_dispatches": ng, "copy_dispatches": nc,
           "strided_copy_check": strided, "command": command}
    out = os.path.join(ROOT, "profiles", f"gla_{kind}_{cfg_key.lower()}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(f"[bench] {out}: {total / 1e6:.1f} MB per launch "
        f"(alg {alg / 1e6:.1f} MB; copy scale fetch {kf:.3f}, write {kw:.3f})")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2", choices=["C1", "C2", "C3", "C4", "CB"])
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough to exceed 512 MB)")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per chunk (0 = the workload's, 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd", action="store_true", help="time gla_bwd (the training backward) instead")
    ap.add_argument("--block", action="store_true", help="time one DiG block forward (DiG-XL/2, C2 grid)")
    ap.add_argument("--order", default="grid", choices=["grid", "zigzag"],
                    help="scan orders: the workload's grid directions, or ZigMa's zigzag tables (GLA only)")
    ap.add_argument("--product-probe", action="store_true",
                    help="only five launches of the block's largest product (for PMC passes)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the launches the PMC passes count: 3 plain copies, 3 gla_fwd")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COMMAND"),
                    help="(no GPU) build the traffic record from the two PMC passes' output folders")
    a = ap.parse_args(argv)

    if a.write_traffic:
        return write_traffic(a.config, *a.write_traffic, bwd=a.bwd)

    if a.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {a.gpus} is not supported "
              "(the path shards by whole (batch, head) units with no communication; run one process per GPU)", file=sys.stderr)
        return 2

    import torch

    from gated_linear_attention_gla_amd import binding as dg
    from gated_linear_attention_gla_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dg.lib()
    if a.product_probe:
        return product_probe()
    if a.traffic_probe:
        return traffic_probe(a.config, a.chunk, bwd=a.bwd)
    if a.bwd:
        return bench_bwd(a, dg, gen, torch)
    if a.block:
        return bench_block(a, dg, gen, torch)
    if a.order == "zigzag":
        return bench_fwd_ordered(a, dg, gen, torch)
    dev = torch.device("cuda:0")
    cfg = gen.CONFIGS[a.config]
    B, T, H, d, C = cfg.B, cfg.T, cfg.H, cfg.d, cfg.C
    grid = (cfg.gh, cfg.gw)
    chunk = a.chunk or cfg.chunk

    ws_bytes = gla_alg_bytes(cfg) + conv_alg_bytes(cfg)
    nsets = a.sets or max(2, math.ceil(512e6 / ws_bytes))
    log(f"[bench] {cfg.key} {cfg.name}: B={B} H={H} T={T} ({cfg.gh}x{cfg.gw}) d={d}; {nsets} input sets")
    sets = []
    for i in range(nsets):
        x = gen.make_inputs(cfg.key, set_index=i, device=dev)
        bufs = {"o": torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev),
                "sf": torch.empty(B, H, d, d, dtype=torch.float32, device=dev),
                "y": torch.empty(B, T, C, dtype=torch.bfloat16, device=dev)}
        if cfg.adaln:
            bufs["m"] = torch.empty_like(x["x_qkv"])
        sets.append((x, bufs))
    nbytes = dg.workspace_bytes(dg.DIG_BF16, B, T, H, d, d, chunk)
    ws = dg.get_workspace(dev, nbytes)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = []

    def step(i, timed=False):
        x, bf = sets[i % nsets]
        direction = cfg.direction(i)
        if cfg.adaln:
            m = dg.adaln_modulate(x["x_qkv"], x["ada_scale"], x["ada_shift"], 1e-6, x["ada_out_scale"], out=bf["m"])
            q, k, v = (m[j].view(B, T, H, d) for j in range(3))
        else:
            q, k, v = x["q"], x["k"], x["v"]
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        dg.gla_fwd(q, k, v, x["log_alpha"], grid, direction, chunk=chunk, out=bf["o"], s_final=bf["sf"],
                   workspace=ws)
        if timed:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            ev.append((e0, e1))
        dg.srem_dwconv(bf["o"].view(B, T, C), x["w"], grid, direction, out=bf["y"])

    # device-copy probe: what a plain read+write stream reaches on this GPU
    # (256 MiB read + 256 MiB written, runtime blit kernel, best of 5)
    csrc = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    copy_ms = []
    for _ in range(6):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        cdst.copy_(csrc)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(c0.elapsed_time(c1))
    copy_gbs = 2 * COPY_PROBE_BYTES / (min(copy_ms[1:]) * 1e-3) / 1e9
    del csrc, cdst

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, bracketed by synchronisation
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(a.steps):
        step(a.warmup + i, timed=True)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / a.steps
    gla_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    gla_avg_ms = sum(gla_ms) / len(gla_ms)
    gla_sorted = sorted(gla_ms)

    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    abytes = gla_alg_bytes(cfg)
    aflops = gla_alg_flops(cfg)
    achieved = abytes / (gla_avg_ms * 1e-3) / 1e9
    traffic = traffic_record(cfg.key)
    log(f"[bench] step {ms_step * 1e3:.1f} us, gla_fwd avg {gla_avg_ms * 1e3:.1f} us "
        f"(median {gla_sorted[len(gla_sorted) // 2] * 1e3:.1f}, p10 {gla_sorted[len(gla_sorted) // 10] * 1e3:.1f}, "
        f"p90 {gla_sorted[(9 * len(gla_sorted)) // 10] * 1e3:.1f}), copy probe {copy_gbs:.0f} GB/s, "
        f"{achieved:.0f} GB/s, wall {wall:.3f} s")

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a bounded sample ...")
        x_cpu = {k_: (v_.cpu() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in sets[0][0].items()}
        cpu = cpu_baseline(cfg, x_cpu)
        log(f"[bench] cpu oracle: {cpu['value']:.3e} tokens/s on {cpu['cores']} cores")

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian activations of the DiG latent-grid shape; no dataset or weights)",
        "config": {"workload": f"{cfg.key} {cfg.name}: GLA fwd (chunk {chunk}, fp32 state) + "
                               f"SREM 3x3 dwconv/remap{', adaLN prologue' if cfg.adaln else ''}",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": d, "grid": list(grid),
                   "directions": list(cfg.dirs), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gla_fwd_bf16_kernel", "alg_bytes_per_launch": abytes,
                     "avg_launch_us": gla_avg_ms * 1e3,
                     "copy_probe_gbs": copy_gbs, "frac_of_copy_probe": achieved / copy_gbs},
        "gla_fwd": {"tokens_per_s": tokens / (gla_avg_ms * 1e-3), "tflops_alg": aflops / (gla_avg_ms * 1e-3) / 1e12,
                    "mfma_frac": aflops / (gla_avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    "median_us": gla_sorted[len(gla_sorted) // 2] * 1e3,
                    "p10_us": gla_sorted[len(gla_sorted) // 10] * 1e3,
                    "p90_us": gla_sorted[(9 * len(gla_sorted)) // 10] * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
