"""The device-side expert cache and the host home for experts, through the C-ABI.

A run of decode steps (different tokens and batch sizes each step) routes, lets
the cache manager rewrite the layer's table, and runs the experts through the
live table.  Every step's outputs must be bit-identical to the same step with
the plain device-resident table (the bytes are the same wherever they are
read), and the manager's hit and miss counts must equal those of the host
policy replay (host/cachesim.c, itself checked against a Python replay) on the
same routing trace, so the victims are the ones the policy defines."""
import numpy as np
import pytest
import torch

import synth
from synth.device import DeviceLayer, x_device
from tests.gpu_util import make_layer_api, say

pytestmark = pytest.mark.gpu

_layers = {}


def _layer(name, dev):
    if name not in _layers:
        _layers[name] = DeviceLayer.generate(synth.CONFIGS[name], 0, dev)
    return _layers[name]


def _host_home(cfg, layer=0):
    """every expert of the layer in one pinned host arena -> (host addr, refs)"""
    import ctypes
    import bit_moe_expert_router_amd as m
    eb = synth.align(synth.expert_bytes(cfg))
    h, d = m.moe_host_arena_create(cfg.n_experts * eb)
    buf = np.ctypeslib.as_array((ctypes.c_uint8 * (cfg.n_experts * eb)).from_address(h))
    off = synth.matrix_offsets(cfg)
    for e in range(cfg.n_experts):
        b = synth.expert_blob(cfg, layer, e)
        buf[e * eb:e * eb + b.size] = b
    refs = [tuple(d + e * eb + o for o in off) for e in range(cfg.n_experts)]
    return h, refs


CASES = [("c2", "lfu", 24, "device"), ("c2", "clock", 24, "device"), ("c1", "lfu", 5, "device"),
         ("c1", "clock", 5, "host"), ("c2", "lfu", 40, "host")]


@pytest.mark.parametrize("name,policy,slots,home", CASES)
def test_cache_steps_bit_identical_and_policy(gpu, name, policy, slots, home):
    import bit_moe_expert_router_amd as m
    from bit_moe_expert_router_amd import cachesim
    cfg = synth.CONFIGS[name]
    say(f"[cache] {name} {policy} S={slots} home={home}")
    dl = _layer(name, gpu)
    Tmax = 4
    ref_ml = make_layer_api(cfg, dl, Tmax)
    ml = make_layer_api(cfg, dl, Tmax)
    host = None
    home_refs = dl.refs
    if home == "host":
        host, home_refs = _host_home(cfg)
    eb = synth.align(synth.expert_bytes(cfg))
    arena = torch.empty(max(slots, 1) * eb, dtype=torch.uint8, device=gpu)
    state = torch.zeros(m.moe_cache_state_bytes(ml.ctx, slots), dtype=torch.uint8, device=gpu)
    decay = 0.9
    pol = m.MOE_CACHE_LFU if policy == "lfu" else m.MOE_CACHE_CLOCK
    m.moe_cache_init(ml.ctx, 0, slots, pol, decay, home_refs, arena, eb, state)
    steps, got_miss = [], []
    rng = np.random.default_rng(5)
    for s in range(30):
        T = int(rng.integers(1, Tmax + 1))
        xh = synth.normal_bf16(T * cfg.hidden, cfg.seed, 100 + s, synth.SYN_X, 1.0).reshape(T, -1)
        xd = torch.from_numpy(xh.view(np.int16)).to(gpu)
        r = ml.route(xd, dl.router, dl.bias)
        m.moe_cache_step(ml.ctx, 0, r.expert_offsets, state)
        out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
        po = torch.empty((T * cfg.top_k, cfg.hidden), dtype=torch.float32, device=gpu)
        ml.forward(0, xd, r, out, po)
        r2 = ref_ml.route(xd, dl.router, dl.bias)
        out2 = torch.empty_like(out)
        po2 = torch.empty_like(po)
        ref_ml.forward(0, xd, r2, out2, po2)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(po, po2), (s, "outputs differ")
        off = r.expert_offsets.cpu().numpy()
        steps.append([np.nonzero(np.diff(off) > 0)[0].tolist()])
        hdr = state[:32].cpu().numpy()  # int64 steps, hits, misses; int32 hits, misses
        got_miss.append(int(hdr[28:32].view(np.int32)[0]))
    tot = state[:24].cpu().numpy().view(np.int64)
    trace, offs, L = cachesim.to_csr(steps)
    ref_miss = cachesim.simulate(trace, offs, L, cfg.n_experts, slots, policy, decay=decay)
    assert got_miss == ref_miss.tolist(), (got_miss, ref_miss.tolist())
    assert tot[0] == 30 and tot[2] == ref_miss.sum() and tot[1] + tot[2] == len(trace)
    say(f"[cache] {name} {policy}: misses per step {got_miss[:12]}..., total {int(tot[2])}")
    ml.close()
    ref_ml.close()
    if host is not None:
        m.moe_host_arena_destroy(host)


def test_host_home_bit_identical(gpu):
    """every expert read zero-copy from pinned host memory gives the outputs of
    the device-resident layer, bit for bit (decode and the matrix-core path)"""
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c2"]
    say("[host home] c2")
    dl = _layer("c2", gpu)
    host, refs = _host_home(cfg)
    for T in (1, 8, 70):
        xh, xd = x_device(cfg, gpu, tokens=T)
        a = make_layer_api(cfg, dl, T)
        b = make_layer_api(cfg, dl, T)
        b.set_table(0, refs)
        outs = []
        for ml in (a, b):
            r = ml.route(xd, dl.router, dl.bias)
            out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
            ml.forward(0, xd, r, out)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), T
        a.close()
        b.close()
    m.moe_host_arena_destroy(host)
