#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer hot path on one MI355X.

A step is one pass of the whole layer (routing: logits, top-k, grouping; experts:
gate/up + SwiGLU, down; shared expert when the workload has one; weighted
combine) over one batch of synthetic tokens whose inputs are already resident in
HBM.  The default workload is one GLM-5.3-Flash-shaped MoE layer at decode batch
1 (hidden 5120, expert intermediate 1536, 288 experts, top-8, 3-bit group-128
weights with bf16 scales, Zipf(1.1) router bias).  Steps rotate over several
resident copies of the layer (distinct weights, router and bias) so that no step
is served from the 256 MB last-level cache.  The timed steps are replays of HIP
graphs that each hold several consecutive layer steps (a decoder replays one graph
over all its layers), so the per-replay launch cost is shared as it is there; every
step in a graph does the whole layer on its own layer's weights.

Prints ONE JSON line: tokens/s over the timed steps, the dominant kernel's
achieved expert-weight bandwidth against the 8 TB/s HBM peak (prefill: matrix-core
flops against the dense fp16 peak; kernel durations from HIP events that each
launch timestamps at the kernel's start and end on its stream), and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 matrix peak of the MI355X
METRIC = "MoE-layer tokens/s (decode b=1..8, prefill 8K) + expert-weight HBM GB/s vs peak"

WORKLOAD_TEXT = {
    "c1": "tiny MoE layer: H 256, I 128, 16 experts, top-2, 4-bit G32 fp16 scales",
    "c2": "one GLM-5.3-Flash-shaped MoE layer at decode: H 5120, I 1536, 288 experts, top-8, "
          "3-bit G128 bf16 scales, Zipf(1.1) router bias",
    "c3": "GLM-shaped MoE layer at decode batch 8 + bf16 shared expert (I 1536), expert pointer "
          "table remapped to a seeded slot permutation, Zipf(1.1) bias",
    "c4": "42-layer stack of GLM-shaped MoE layers at decode batch 4 (RMSNorm glue, shared experts, "
          "remapped tables, own Zipf bias per layer)",
    "c5": "8,192-token prefill chunk through one GLM-shaped MoE layer (3-bit G128), Zipf(1.1) bias",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--tokens", type=int, default=None, help="batch (default: the workload's)")
    ap.add_argument("--uniform", action="store_true", help="no Zipf router bias")
    ap.add_argument("--layers", type=int, default=None,
                    help="resident layer copies the steps rotate over (default: 16 at decode)")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--graph-steps", type=int, default=8,
                    help="consecutive layer steps captured in one HIP graph for the single-layer "
                         "workloads (as a decoder replays one graph over many layers); the largest "
                         "value up to this that divides both --steps and the rotated layer count")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle baseline sample (0: skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--no-kernel-timing", action="store_true")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; a multi-GPU run is not part of it "
                                   "(expert or data parallel sharding is described in DESIGN.md)",
                          "n_gpus": a.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth.device import DeviceLayer
    import bit_moe_expert_router_amd as moe

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[a.workload]
    if a.tokens:
        cfg = cfg.with_(tokens=a.tokens)
    if a.uniform:
        cfg = cfg.with_(zipf=False)
    T = cfg.tokens
    decode = T <= 64
    stack = cfg.layers > 1
    L = cfg.layers if stack else (a.layers or (16 if decode else 1))

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
        from bit_moe_expert_router_amd.layer import stack_forward
        resid = torch.from_numpy(
            synth.normal_f32(T * cfg.hidden, cfg.seed, 0, synth.SYN_X, 1.0).reshape(T, cfg.hidden)).to(dev)
        ybuf = torch.empty((T, cfg.hidden), dtype=torch.int16, device=dev)
        routers = [dl.router for dl in layers]
        biases = [dl.bias for dl in layers]

    def step(l):
        if stack:  # one pass through every layer of the stack
            stack_forward(ml, resid, out, routers, biases, ybuf, out)
            return
        dl = layers[l]
        r = ml.route(xd, dl.router, dl.bias)
        ml.forward(l, xd, r, out)

    # distinct experts per layer (deterministic: same x, same layer -> same routing)
    U = []
    if stack:
        out.zero_()
        seen = []
        stack_forward(ml, resid, out, routers, biases, ybuf, out,
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
    eb = synth.expert_bytes(cfg)
    glay, ulay, dlay = synth.expert_layouts(cfg)
    kern = {}
    kt_steps = min(a.steps, 10) if stack else a.steps
    if not a.no_kernel_timing:
        moe.moe_profile_read()  # drop anything recorded before
        moe.moe_profile_enable(True)
        for i in range(kt_steps):
            step(i % L)
        torch.cuda.synchronize()
        moe.moe_profile_enable(False)
        kern = moe.moe_profile_read()
    # algorithmic bytes over the kernel-timing pass (same step sequence); a stack
    # step launches every layer once
    u_steps = [U[i % L] for i in range(kt_steps)] if not stack else [u for _ in range(kt_steps) for u in U]
    gu_bytes = sum(u * (glay.nbytes + ulay.nbytes) for u in u_steps)
    dn_bytes = sum(u * dlay.nbytes for u in u_steps)
    roof = None
    extra = {}
    prefill = T > 64 and cfg.hidden % 128 == 0 and cfg.inter % 128 == 0
    # algorithmic matrix-core work of the prefill path: every pair's gate and up
    # products (2 x 2*H*I flops) and its down product (2*I*H flops)
    gu_flops = T * cfg.top_k * 4 * cfg.hidden * cfg.inter
    dn_flops = T * cfg.top_k * 2 * cfg.hidden * cfg.inter
    if kern:
        gu_ms, gu_n = kern.get("gateup", (0.0, 0))
        dn_ms, dn_n = kern.get("down", (0.0, 0))
        if prefill:
            ach = gu_flops * gu_n / (gu_ms * 1e-3) / 1e12 if gu_ms else None
            roof = {"bound": "mfma", "achieved": round(ach, 1) if ach else None,
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4) if ach else None,
                    "traffic": measured_traffic("k_gateup_mfma", a.workload),
                    "kernel": "k_gateup_mfma (grouped gate+up GEMM, SwiGLU epilogue)",
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                    "avg_us": round(gu_ms / gu_n * 1e3, 2) if gu_n else None,
                    "flops_per_launch": gu_flops}
            if dn_ms:
                extra["down_TFLOPs"] = round(dn_flops * dn_n / (dn_ms * 1e-3) / 1e12, 1)
        else:
            ach = gu_bytes / (gu_ms * 1e-3) / 1e9 if gu_ms else None
            gu_kernel = "k_gateup_smem" if T <= 2 else "k_gemv (gate/up)"
            roof = {"bound": "hbm", "achieved": round(ach, 1) if ach else None, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4) if ach else None,
                    "traffic": measured_traffic(gu_kernel, a.workload),
                    "kernel": gu_kernel + " (gate and up GEMV)",
                    "avg_us": round(gu_ms / gu_n * 1e3, 2) if gu_n else None,
                    "bytes_per_launch": round(gu_bytes / len(u_steps)),
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"}
            if dn_ms:
                extra["down_GBs"] = round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1)
        extra["kernels_us"] = {k: round(v[0] / v[1] * 1e3, 2) for k, v in kern.items() if v[1]}
        tot_ms = sum(v[0] for v in kern.values())
        extra["expert_bytes_per_step"] = round((gu_bytes + dn_bytes) / kt_steps)
        extra["expert_GBs_over_kernel_time"] = round((gu_bytes + dn_bytes) / (tot_ms * 1e-3) / 1e9, 1)
    extra["expert_GBs_over_step"] = round((gu_bytes + dn_bytes) / kt_steps / (ms_step * 1e-3) / 1e9, 1)
    extra["distinct_experts_per_step"] = round(float(np.mean(u_steps)), 2)
    extra["graph_replay"] = graphs is not None
    extra["steps_per_graph"] = G if graphs is not None else None
    extra["input_gen_s"] = round(gen_s, 1)

    if a.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        extra["calib_copy_bytes"] = 1 << 30

    # ---------------------------------------------------------- CPU oracle baseline
    cpu = None
    if a.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, L, a.cpu_seconds, layers_per_step=L if stack else 1)

    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if prefill else "bf16",
        "data": "synthetic (seeded counter-based generator; random 3-bit codes and scales, "
                "N(0,1) bf16 activations, N(0,0.02) fp32 router)",
        "config": {"workload": f"{a.workload}: {WORKLOAD_TEXT[a.workload]}", "tokens": T,
                   "layers_rotated": L, "hidden": cfg.hidden, "inter": cfg.inter,
                   "experts": cfg.n_experts, "top_k": cfg.top_k, "bits": cfg.bits,
                   "group": cfg.group, "zipf": cfg.zipf, "shared_inter": cfg.shared_inter},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(res))
    ml.close()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated against a
    plain device copy), or None when there is none for this workload or the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        ent = json.load(fh).get("kernels", {}).get(kernel)
    if not ent or ent.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for src in ent["sources"]:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != ent["sha256_16"]:
        return None
    return ent["hbm_bytes_per_launch"]


def cpu_baseline(cfg, L, budget_s, layers_per_step=1):
    """fp64 oracle (the test reference, untuned) on the host cores: routing, every
    pick's expert FFN and the combine of one batch per layer, rotating over the
    same layers; timed until the budget is spent.  Batches above 16 tokens are
    sampled: the first 16 tokens of the batch are routed and computed per layer.
    A step of a stack is layers_per_step such layers."""
    import numpy as np

    import oracle
    import synth

    off = synth.matrix_offsets(cfg)
    T = min(cfg.tokens, 16)
    xh = synth.x_bf16(cfg)[:T]
    cache = {}
    steps, spent = 0, 0.0
    while spent < budget_s:
        l = steps % L
        if l not in cache:
            wr, bias = synth.router_f32(cfg, l), synth.zipf_bias(cfg, l)
            ids, _, _, _ = oracle.route(xh, wr, bias, cfg.top_k)
            blobs = {int(e): synth.expert_blob(cfg, l, int(e)) for e in np.unique(ids)}
            tabs = [[blobs[e][off[m]:(off[m + 1] if m < 2 else None)] if e in blobs else
                     np.zeros(16, np.uint8) for e in range(cfg.n_experts)] for m in range(3)]
            cache[l] = (wr, bias, tabs, synth.shared_weights(cfg, l))
        wr, bias, tabs, shared = cache[l]
        t0 = time.perf_counter()  # input generation above is not timed
        ids, w, _, _ = oracle.route(xh, wr, bias, cfg.top_k)
        oracle.moe_layer(xh, ids, w, *tabs, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16, shared)
        spent += time.perf_counter() - t0
        steps += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(T * steps / spent / layers_per_step, 3), "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{steps} layer evaluations of {T} token(s) of the same workload (routing + "
                      f"every pick's fp64 expert FFN + combine, rotating over {min(L, steps)} "
                      f"layers; a step is {layers_per_step} layer(s)), {spent:.1f} s, "
                      f"{threads} OpenMP threads"}


if __name__ == "__main__":
    main()
