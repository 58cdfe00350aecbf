#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer hot path on one MI355X.

A step is one pass of the whole layer (routing: logits, top-k, grouping; experts:
gate/up + SwiGLU, down; shared expert when the workload has one; weighted
combine) over one batch of synthetic tokens whose inputs are already resident in
HBM.  The headline workload is one GLM-5.3-Flash-shaped MoE layer at decode batch
1 (hidden 5120, expert intermediate 1536, 288 experts, top-8, 3-bit group-128
weights with bf16 scales, Zipf(1.1) router bias).  Decode steps rotate over
several resident copies of the layer (distinct weights, router and bias) so that
no step is served from the 256 MB last-level cache.  The timed steps are replays
of HIP graphs that each hold several consecutive layer steps (a decoder replays
one graph over all its layers), so the per-replay launch cost is shared as it is
there; every step in a graph does the whole layer on its own layer's weights.

Prints ONE JSON line.  `value` is the headline workload's tokens/s.  `roofline`
describes the longest kernel of its step: algorithmic expert-weight bytes per
launch over the kernel's average duration against the 8 TB/s HBM peak (prefill:
matrix-core flops against the dense fp16 peak), with durations from HIP events
that each launch timestamps at the kernel's start and end on its own stream (the
average of a kernel's launches within twice their median: an event pair is now
and then held back by the host side of a launch; raw means and medians are given
too), and
the HBM traffic rocprofv3 counted for that kernel (when the committed counter
summary matches the current sources).  `extra.step` gives the whole step's
expert bytes over the step time.  `extra.workloads` repeats all of this for the
decode batch sweep (2, 4, 8 tokens), batch 8 with the shared expert and remapped
table, the 42-layer stack at batch 4 and the 8,192-token prefill chunk with Zipf
and uniform routing.  `cpu_baseline` is the fp64 CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 matrix peak of the MI355X
MFMA_F64_PEAK_TFLOPS = 78.6    # dense fp64 matrix peak
METRIC = "MoE-layer tokens/s (decode b=1..8, prefill 8K) + expert-weight HBM GB/s vs peak"

WORKLOADS = {
    "c1": ("c1", {}, "tiny MoE layer: H 256, I 128, 16 experts, top-2, 4-bit G32 fp16 scales"),
    "c2": ("c2", {}, "one GLM-5.3-Flash-shaped MoE layer at decode batch 1: H 5120, I 1536, "
                     "288 experts, top-8, 3-bit G128 bf16 scales, Zipf(1.1) router bias"),
    "c2b2": ("c2", {"tokens": 2}, "the same layer at decode batch 2"),
    "c2b4": ("c2", {"tokens": 4}, "the same layer at decode batch 4"),
    "c2b8": ("c2", {"tokens": 8}, "the same layer at decode batch 8"),
    "c3": ("c3", {}, "GLM-shaped MoE layer at decode batch 8 + bf16 shared expert (I 1536), expert "
                     "pointer table remapped to a seeded slot permutation, Zipf(1.1) bias"),
    "c4": ("c4", {}, "42-layer stack of GLM-shaped MoE layers at decode batch 4 (RMSNorm glue, "
                     "shared experts, remapped tables, own Zipf bias per layer)"),
    "c5": ("c5", {}, "8,192-token prefill chunk through one GLM-shaped MoE layer (3-bit G128), "
                     "Zipf(1.1) bias"),
    "c5u": ("c5", {"zipf": False}, "8,192-token prefill chunk through one GLM-shaped MoE layer "
                                   "(3-bit G128), uniform routing (no bias)"),
    "q2": ("q2", {}, "the GLM-shaped layer at decode batch 1 with 2-bit codes in groups of 128 "
                     "(2.125 bits per weight), Zipf(1.1) bias"),
    "q2b8": ("q2", {"tokens": 8}, "the 2-bit layer at decode batch 8"),
    "q4": ("q4", {}, "the GLM-shaped layer at decode batch 1 with 4-bit codes in groups of 128 "
                     "(4.125 bits per weight), Zipf(1.1) bias"),
    "q4b8": ("q4", {"tokens": 8}, "the 4-bit layer at decode batch 8"),
}
DEFAULT_EXTRA = "c2b2,c2b4,c2b8,c3,c4,c5,c5u,q2,q2b8,q4,q4b8"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated further workloads reported under extra.workloads "
                         "('' for none)")
    ap.add_argument("--tokens", type=int, default=None, help="batch of the main workload")
    ap.add_argument("--layers", type=int, default=None,
                    help="resident layer copies the decode steps rotate over (default 20)")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--layer-calls", choices=("fused", "split"), default="fused",
                    help="single-layer workloads: one moe_layer_forward call per step (fused) or "
                         "moe_route then moe_forward (split)")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="consecutive layer steps captured in one HIP graph for the single-layer "
                         "workloads (as a decoder replays one graph over many layers); the largest "
                         "value up to this that divides both --steps and the rotated layer count")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the main workload's CPU-oracle baseline (0: skip); the further "
                         "workloads get a quarter of it each")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-cache", action="store_true",
                    help="skip the host-home / expert-cache measurement and the policy replay")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--stack-calls", choices=("fused", "three"), default="fused",
                    help="stack workloads: one moe_stack_layer call per layer (default), or "
                         "moe_rmsnorm_bf16 + moe_route + moe_forward")
    return ap.parse_args()


# ------------------------------------------------------------------ work per kernel
def kernel_symbol(kname, T, prefill):
    """library kernel behind a profiled name at batch T"""
    if prefill:
        return {"gateup": "k_gateup_mfma", "down": "k_down_mfma", "route_logits": "k_logits_mfma",
                "combine": "k_combine"}.get(kname, kname)
    if T <= 2:
        return {"gateup": "k_gateup_smem", "down": "k_down_blk", "route": "k_route_small",
                "combine": "k_combine_parts"}.get(kname, kname)
    return {"gateup": "k_gemv<MODE 0> (gate/up)", "down": "k_gemv_mma<MODE 1> (down)",
            "route_logits": "k_logits_multi", "combine": "k_combine_parts",
            "swiglu": "k_swiglu_sum", "plan": "k_plan_decode",
            "shared_gateup": "k_shared_gateup", "shared_down": "k_shared_down"}.get(kname, kname)


def kernel_work(kname, cfg, T, u_mean, lay, prefill):
    """(algorithmic amount per launch, kind) of a profiled kernel; kind is "bytes",
    "f16" (matrix-core flops) or "f64" (fp64 matrix-core flops); None for the
    latency-bound glue kernels"""
    glay, ulay, dlay = lay
    P = T * cfg.top_k
    H, I, E, Is = cfg.hidden, cfg.inter, cfg.n_experts, cfg.shared_inter
    if kname == "gateup":
        return (4 * P * H * I, "f16") if prefill else (u_mean * (glay.nbytes + ulay.nbytes), "bytes")
    if kname == "down":
        return (2 * P * H * I, "f16") if prefill else (u_mean * dlay.nbytes, "bytes")
    if kname == "route":
        return E * H * 4 + T * H * 2, "bytes"
    if kname == "route_logits":
        return (2 * T * E * H, "f64") if T > 32 else (E * H * 4 + T * H * 2, "bytes")
    if kname == "shared_gateup":
        return 2 * Is * H * 2, "bytes"
    if kname == "shared_down":
        return H * Is * 2, "bytes"
    return None


def roofline_of(kname, avg_us, work, traffic):
    amount, kind = work
    if kind == "bytes":
        ach = amount / (avg_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "bytes_per_launch": round(amount)}
    peak = MFMA_F16_PEAK_TFLOPS if kind == "f16" else MFMA_F64_PEAK_TFLOPS
    ach = amount / (avg_us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "traffic": traffic, "flops_per_launch": round(amount),
            "dtype": "f16" if kind == "f16" else "f64"}


def measured_traffic(symbol, workload):
    """HBM bytes per launch of `symbol` on `workload` from the committed counter
    summary (profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated
    against a plain device copy), or None when there is none or the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        ent = json.load(fh).get("kernels", {}).get(f"{symbol}@{workload}")
    if not ent:
        return None
    h = hashlib.sha256()
    for src in ent["sources"]:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != ent["sha256_16"]:
        return None
    return ent["hbm_bytes_per_launch"]


# ------------------------------------------------------------------ one workload
def run_workload(name, a, dev, cpu_budget, cpu_jobs, main_tokens=None, one_thread=True):
    import numpy as np
    import torch

    import synth
    from synth.device import DeviceLayer
    import bit_moe_expert_router_amd as moe

    base, over, text = WORKLOADS[name]
    cfg = synth.CONFIGS[base].with_(**over)
    if main_tokens:
        cfg = cfg.with_(tokens=main_tokens)
    T = cfg.tokens
    decode = T <= 64
    stack = cfg.layers > 1
    L = cfg.layers if stack else ((a.layers or 20) if decode else 1)
    prefill = T > 64 and cfg.hidden % 128 == 0 and cfg.inter % 128 == 0

    # ---------------------------------------------------------- resident inputs
    t0 = time.time()
    layers = [DeviceLayer.generate(cfg, l, dev) for l in range(L)]
    xh = synth.x_bf16(cfg)
    xd = torch.from_numpy(xh.view(np.int16)).to(dev)
    ml = moe.MoELayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits, cfg.group,
                      cfg.scale_f16, cfg.shared_inter, T, L, dev)
    for l, dl in enumerate(layers):
        ml.set_table(l, dl.refs)
        if dl.shared is not None:
            ml.set_shared(l, *dl.shared)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    if stack:
        from bit_moe_expert_router_amd.layer import stack_forward, stack_forward_fused
        resid = torch.from_numpy(
            synth.normal_f32(T * cfg.hidden, cfg.seed, 0, synth.SYN_X, 1.0).reshape(T, cfg.hidden)).to(dev)
        ybuf = torch.empty((T, cfg.hidden), dtype=torch.int16, device=dev)
        routers = [dl.router for dl in layers]
        biases = [dl.bias for dl in layers]

    def step(l):
        if stack:  # one pass through every layer of the stack
            if a.stack_calls == "fused":
                stack_forward_fused(ml, resid, routers, biases, ybuf, out)
            else:
                stack_forward(ml, resid, out, routers, biases, ybuf, out)
            return
        dl = layers[l]
        if a.layer_calls == "fused":  # moe_layer_forward: routing and experts in one call
            ml.layer_forward(l, xd, dl.router, dl.bias, out)
        else:
            r = ml.route(xd, dl.router, dl.bias)
            ml.forward(l, xd, r, out)

    # distinct experts per layer (deterministic: same x, same layer -> same routing)
    U = []
    if stack:
        out.zero_()
        seen = []
        stack_forward_fused(ml, resid, routers, biases, ybuf, out,
                            on_layer=lambda l, y_, r, o_: seen.append(r.expert_offsets.clone()))
        torch.cuda.synchronize()
        U = [int((np.diff(o.cpu().numpy()) > 0).sum()) for o in seen]
    else:
        for l in range(L):
            step(l)
            torch.cuda.synchronize()
            off = ml.rb.expert_offsets.cpu().numpy()
            U.append(int((np.diff(off) > 0).sum()))

    # G consecutive steps per graph (a stack step is already a whole pass)
    G = 1
    if not stack and not a.eager:
        G = max(1, min(a.graph_steps, L, a.steps))
        while a.steps % G or L % G:
            G -= 1
    graphs = None
    if not a.eager:
        graphs = []
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for l in range(1 if stack else L):
                step(l)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for j in range(1 if stack else L // G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    step(j * G + i)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):  # steps i .. i+G-1
        if graphs is not None:
            graphs[(i // G) % len(graphs)].replay()
        else:
            step(i % L)

    for i in range(0, max(a.warmup, G), G):
        run(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for i in range(0, a.steps, G):
        run(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / a.steps
    tokens_per_s = T * a.steps / wall

    # ---------------------------------------------------------- kernel timing
    lay = synth.expert_layouts(cfg)
    kern = {}
    kt_steps = min(a.steps, 10) if stack else a.steps
    if not a.no_kernel_timing:
        # one untimed eager pass first: the timing pass then starts from the same
        # warm state as the steps before it
        for i in range(kt_steps):
            step(i % L)
        torch.cuda.synchronize()
        moe.moe_profile_read()  # drop anything recorded before
        moe.moe_profile_enable(True)
        for i in range(kt_steps):
            step(i % L)
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        kern = moe.moe_profile_read_stats()
    # algorithmic bytes over the kernel-timing pass (same step sequence); a stack
    # step launches every layer once
    u_steps = [U[i % L] for i in range(kt_steps)] if not stack else [u for _ in range(kt_steps) for u in U]
    u_mean = float(np.mean(u_steps))
    expert_bytes_step = sum(u_steps) * synth.expert_bytes(cfg) / kt_steps
    shared_bytes_step = (L if stack else 1) * synth.shared_bytes(cfg)
    res = {"workload": f"{name}: {text}", "tokens": T, "value": round(tokens_per_s, 1),
           "unit": "tokens/s", "ms_per_step": round(ms_step, 5),
           "distinct_experts_per_layer": round(u_mean, 2), "layers_rotated": L,
           "graph_replay": graphs is not None, "steps_per_graph": G if graphs is not None else None,
           "input_gen_s": round(gen_s, 1)}
    if stack:
        res["stack_calls"] = ("one moe_stack_layer call per layer" if a.stack_calls == "fused"
                              else "moe_rmsnorm_bf16 + moe_route + moe_forward per layer")
    roof = None
    if kern:
        # a kernel's duration: the mean of its launches within twice their median (an
        # event pair is occasionally held back by the host side of a launch)
        us = {k: v[2] * 1e3 for k, v in kern.items() if v[3]}
        per_step_us = {k: us[k] * kern[k][3] / kt_steps for k in us}
        res["kernels_us"] = {k: round(v, 2) for k, v in us.items()}
        res["kernels_us_median"] = {k: round(kern[k][1] * 1e3, 2) for k in us}
        res["kernels_us_raw_mean"] = {k: round(kern[k][0] / kern[k][3] * 1e3, 2) for k in us}
        # the longest kernel of the step (time per step), with its own roofline
        ranked = sorted(per_step_us, key=lambda k: -per_step_us[k])
        for k in ranked:
            work = kernel_work(k, cfg, T, u_mean, lay, prefill)
            if work is None:
                continue
            sym = kernel_symbol(k, T, prefill)
            roof = roofline_of(k, us[k], work, measured_traffic(sym, name))
            roof.update({"kernel": sym, "avg_us": round(us[k], 2),
                         "longest_in_step": k == ranked[0],
                         "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                         "calibrated against a plain device copy)"})
            break
        others = {}
        for k in ranked:
            work = kernel_work(k, cfg, T, u_mean, lay, prefill)
            if work is not None and (roof is None or kernel_symbol(k, T, prefill) != roof["kernel"]):
                r = roofline_of(k, us[k], work, None)
                others[k] = {"achieved": r["achieved"], "unit": r["unit"], "frac": r["frac"]}
        res["other_kernels_roofline"] = others
    step_bytes = expert_bytes_step + shared_bytes_step
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    res["step"] = {"expert_bytes": round(step_bytes), "achieved_GBs": round(step_gbs, 1),
                   "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                   "note": "routed expert bytes (once per distinct expert per layer) + shared "
                           "expert bytes, over the whole step time"}
    if prefill:
        flops = 6 * T * cfg.top_k * cfg.hidden * cfg.inter
        tf = flops / (ms_step * 1e-3) / 1e12
        res["step"].update({"flops": flops, "achieved_TFLOPs": round(tf, 1),
                            "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
    res["roofline"] = roof
    res["dtype"] = "f16" if prefill else "bf16"

    # release the device memory before the CPU leg and the next workload
    del graphs, layers, xd, out
    ml.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if cpu_budget > 0:  # run after every GPU measurement (busy host threads slow the launches)
        cpu_jobs.append((res, (cfg, L, cpu_budget), dict(layers_per_step=L if stack else 1,
                                                         one_thread=one_thread)))
    return res


def _ar1_tokens(cfg, n, rho, seed):
    """n bf16 tokens whose N(0,1) entries follow x_t = rho x_{t-1} + sqrt(1-rho^2) e_t
    (consecutive decode tokens are alike): synthetic inputs for routing traces"""
    import numpy as np
    import synth
    eps = synth.normal_f32(n * cfg.hidden, cfg.seed, seed, synth.SYN_X, 1.0).reshape(n, -1)
    x = np.empty_like(eps)
    x[0] = eps[0]
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, n):
        x[t] = rho * x[t - 1] + c * eps[t]
    return synth.bf16_bits(x)


def cache_report(dev, steps=64):
    """Decode of one GLM-shaped layer (batch 1, Zipf routing) with every expert in
    a pinned host arena: read zero-copy alone, and through the device-side LFU
    cache of 64 slots; beside the same token sequence with the layer in HBM.  Plus
    misses per token of the five policies on a routing trace of the 42-layer
    stack's routers (the library's own routing of correlated synthetic tokens),
    replayed by the host tool."""
    import numpy as np
    import torch
    import synth
    import bit_moe_expert_router_amd as moe
    from bit_moe_expert_router_amd import cachesim
    from synth.device import DeviceLayer
    cfg = synth.CONFIGS["c2"]
    res = {}
    dl = DeviceLayer.generate(cfg, 0, dev)
    eb = synth.align(synth.expert_bytes(cfg))
    import ctypes
    h, d = moe.moe_host_arena_create(cfg.n_experts * eb)
    try:
        buf = np.ctypeslib.as_array((ctypes.c_uint8 * (cfg.n_experts * eb)).from_address(h))
        off = synth.matrix_offsets(cfg)
        for e in range(cfg.n_experts):
            b = synth.expert_blob(cfg, 0, e)
            buf[e * eb:e * eb + b.size] = b
        host_refs = [tuple(d + e * eb + o for o in off) for e in range(cfg.n_experts)]
        xs = torch.from_numpy(_ar1_tokens(cfg, steps, 0.95, 7).view(np.int16)).to(dev)
        S = 64
        arena = torch.empty(S * eb, dtype=torch.uint8, device=dev)

        def run(mode):
            ml = moe.MoELayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits,
                              cfg.group, cfg.scale_f16, 0, 1, 1, dev)
            state = None
            if mode == "hbm":
                ml.set_table(0, dl.refs)
            elif mode == "zero_copy":
                ml.set_table(0, host_refs)
            else:
                state = torch.zeros(moe.moe_cache_state_bytes(ml.ctx, S), dtype=torch.uint8,
                                    device=dev)
                moe.moe_cache_init(ml.ctx, 0, S, moe.MOE_CACHE_LFU, 0.995, host_refs, arena, eb,
                                   state)
            out = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for t in range(steps):
                x = xs[t:t + 1]
                r = ml.route(x, dl.router, dl.bias)
                if state is not None:
                    moe.moe_cache_step(ml.ctx, 0, r.expert_offsets, state)
                ml.forward(0, x, r, out)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            r = {"tokens_per_s": round(1e3 / ms, 1), "ms_per_token": round(ms, 4)}
            if state is not None:
                hdr = state[:24].cpu().numpy().view(np.int64)
                r.update({"slots": S, "misses_per_token": round(float(hdr[2]) / steps, 2),
                          "hit_rate": round(float(hdr[1]) / float(hdr[1] + hdr[2]), 3)})
            ml.close()
            return r

        for mode in ("hbm", "zero_copy", "lfu_cache"):
            res[mode] = run(mode)
        res["note"] = ("batch 1, Zipf(1.1) routing, one layer, a run of correlated synthetic "
                       f"tokens (rho 0.95), {steps} steps from a cold cache, eager launches; "
                       "home = pinned host arena read over the host link")
    finally:
        moe.moe_host_arena_destroy(h)
    del dl
    torch.cuda.empty_cache()

    # policy replay on a 42-layer routing trace
    c4 = synth.CONFIGS["c4"]
    ntok = 512
    pol = {}
    for rho in (0.0, 0.95):
        steps_l = [[None] * c4.layers for _ in range(ntok)]
        ml = moe.MoELayer(c4.hidden, c4.inter, c4.n_experts, c4.top_k, c4.bits, c4.group,
                          c4.scale_f16, 0, ntok, 1, dev)
        for l in range(c4.layers):
            x = torch.from_numpy(_ar1_tokens(c4, ntok, rho, 1000 + l).view(np.int16)).to(dev)
            wr = torch.from_numpy(synth.router_f32(c4, l)).to(dev)
            b = torch.from_numpy(synth.zipf_bias(c4, l)).to(dev)
            r = ml.route(x, wr, b)
            ids = r.topk_ids.cpu().numpy()
            for t in range(ntok):
                steps_l[t][l] = ids[t].tolist()
        ml.close()
        trace, offs, L = cachesim.to_csr(steps_l)
        row = {}
        for S in (40, 80, 170):
            row[str(S)] = {p_: round(float(cachesim.simulate(trace, offs, L, c4.n_experts, S, p_,
                                                              0.995).sum()) / ntok, 2)
                           for p_ in ("static", "lru", "lfu", "belady", "clock")}
        pol[f"rho_{rho}"] = row
    res["policy_misses_per_token"] = pol
    res["policy_note"] = (f"{ntok} decode tokens at batch 1 through the 42 layers' routers (own "
                          "Zipf bias each), tokens correlated step to step with coefficient rho; "
                          "slots per layer; the host replay of host/cachesim.c")
    return res


def stream_ceiling(dev):
    """The practical HBM read rate for a launch of the decode kernels' sizes: the
    library's streaming-read probe (moe_stream_read: the weight stream's access
    pattern, 16-byte loads, each wave instruction on 1,024 contiguous bytes) over
    rotating distinct buffers (no last-level-cache reuse), its kernel-own
    duration from the library's HIP-event timing; plus a torch copy for
    reference."""
    import torch
    import bit_moe_expert_router_amd as moe
    res = {}
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    for mb in (24.576, 49.152, 73.728, 1073.741824):
        nbytes = int(mb * 1e6) // 16 * 16
        nbuf = max(2, int(600e6 // nbytes) + 1)
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(nbuf)]
        reps = max(2 * nbuf, 8)
        for b in bufs:
            moe.moe_stream_read(b, nbytes, sink)
        torch.cuda.synchronize()
        moe.moe_profile_read()
        moe.moe_profile_enable(True)
        for i in range(reps):
            moe.moe_stream_read(bufs[i % nbuf], nbytes, sink)
        torch.cuda.synchronize()
        prof = moe.moe_profile_read_stats()
        moe.moe_profile_enable(False)
        rd_us = prof["stream_read"][2] * 1e3  # mean of the launches within twice the median
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            dst.copy_(bufs[i % nbuf])
        e1.record()
        torch.cuda.synchronize()
        cp_us = e0.elapsed_time(e1) * 1e3 / reps
        res[f"{mb:.1f}MB"] = {"read_us": round(rd_us, 2), "read_GBs": round(nbytes / rd_us / 1e3, 1),
                              "copy_us": round(cp_us, 2),
                              "copy_GBs_read_plus_write": round(2 * nbytes / cp_us / 1e3, 1)}
        del bufs, dst
        torch.cuda.empty_cache()
    res["how"] = ("read: the library's streaming-read probe (moe_stream_read) over rotating "
                  "distinct buffers, kernel-own durations from its HIP-event timing; copy: "
                  "torch copy_ (read + write), HIP events around back-to-back launches")
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, L, budget_s, layers_per_step=1, one_thread=True):
    """fp64 oracle (the test reference, untuned) on the host cores: routing, every
    pick's expert FFN and the combine of one batch per layer, rotating over the
    same layers.  Batches above 16 tokens are sampled: the first 16 tokens of the
    batch are routed and computed per layer.  Three timed runs at the host's full
    OpenMP thread count (median reported) and three at one thread on a one-token
    sample; each run does at least one layer evaluation.  A step of a stack is
    layers_per_step such layers."""
    import numpy as np

    import oracle
    import synth

    off = synth.matrix_offsets(cfg)
    cache = {}

    def layer_inputs(l):
        if l not in cache:
            wr, bias = synth.router_f32(cfg, l), synth.zipf_bias(cfg, l)
            xs = synth.x_bf16(cfg)[:min(cfg.tokens, 16)]
            ids, _, _, _ = oracle.route(xs, wr, bias, cfg.top_k)
            blobs = {int(e): synth.expert_blob(cfg, l, int(e)) for e in np.unique(ids)}
            tabs = [[blobs[e][off[m]:(off[m + 1] if m < 2 else None)] if e in blobs else
                     np.zeros(16, np.uint8) for e in range(cfg.n_experts)] for m in range(3)]
            cache[l] = (wr, bias, tabs, synth.shared_weights(cfg, l))
        return cache[l]

    def timed(T, budget, start):
        xh = synth.x_bf16(cfg)[:T]
        steps, spent = 0, 0.0
        while spent < budget or steps == 0:
            l = (start + steps) % L
            wr, bias, tabs, shared = layer_inputs(l)
            t0 = time.perf_counter()  # input generation above is not timed
            ids, w, _, _ = oracle.route(xh, wr, bias, cfg.top_k)
            oracle.moe_layer(xh, ids, w, *tabs, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16,
                             shared)
            spent += time.perf_counter() - t0
            steps += 1
        return T * steps / spent / layers_per_step, steps, spent

    nthr = oracle.max_threads()
    T = min(cfg.tokens, 16)
    all_runs = [timed(T, budget_s / (4 if one_thread else 3), 3 * i) for i in range(3)]
    one_runs = []
    if one_thread:
        oracle.set_threads(1)
        try:
            one_runs = [timed(1, budget_s / 12, 3 * i) for i in range(3)]
        finally:
            oracle.set_threads(nthr)
    v_all = statistics.median(r[0] for r in all_runs)
    res = {"value": round(v_all, 3), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
           "cpu_model": cpu_model(), "nproc": os.cpu_count(),
           "sample": f"median of 3 runs of {'/'.join(str(r[1]) for r in all_runs)} layer "
                     f"evaluations of {T} token(s) of the same workload (routing + every pick's "
                     f"fp64 expert FFN + combine, rotating over the layers; a step is "
                     f"{layers_per_step} layer(s)) at {nthr} OpenMP threads"}
    if one_runs:
        res["one_thread"] = round(statistics.median(r[0] for r in one_runs), 4)
        res["sample"] += (f"; one_thread: median of 3 runs of "
                          f"{'/'.join(str(r[1]) for r in one_runs)} one-token evaluations at 1 thread")
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; a multi-GPU run is not part of it "
                                   "(expert or data parallel sharding is described in DESIGN.md)",
                          "n_gpus": a.gpus}))
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    cpu_jobs = []
    main_res = run_workload(a.workload, a, dev, a.cpu_seconds, cpu_jobs, main_tokens=a.tokens)
    print(f"[bench] {a.workload}: {main_res['value']} tokens/s", file=sys.stderr, flush=True)
    extra = {}
    for name in [w for w in a.extra.split(",") if w and w != a.workload]:
        extra[name] = run_workload(name, a, dev, a.cpu_seconds / 4, cpu_jobs, one_thread=False)
        print(f"[bench] {name}: {extra[name]['value']} tokens/s", file=sys.stderr, flush=True)
    ceiling = None if a.no_ceiling else stream_ceiling(dev)
    cache = None if a.no_cache else cache_report(dev)
    for res_w, args, kw in cpu_jobs:  # the CPU oracle baselines, after all GPU work
        res_w["cpu_baseline"] = cpu_baseline(*args, **kw)

    if a.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    m = main_res
    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic (seeded counter-based generator; random 3-bit codes and scales, "
                "N(0,1) bf16 activations, N(0,0.02) fp32 router)",
        "config": {"workload": m["workload"], "tokens": m["tokens"],
                   "layers_rotated": m["layers_rotated"]},
        "roofline": m["roofline"],
        "cpu_baseline": m.get("cpu_baseline"),
        "extra": {k: v for k, v in m.items() if k not in ("roofline", "cpu_baseline", "value",
                                                           "ms_per_step", "dtype", "unit")},
    }
    res["extra"]["workloads"] = extra
    res["extra"]["stream_ceiling"] = ceiling
    res["extra"]["cache"] = cache
    if a.calib_copy:
        res["extra"]["calib_copy_bytes"] = 1 << 30
    print(json.dumps(res))


if __name__ == "__main__":
    main()
