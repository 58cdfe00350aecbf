"""HIP path vs the fp64 oracle on the same seeded bytes, through the C-ABI.

Routing ids, offsets, sorted pairs and pair positions must match bit-exactly;
every expert output y(t,k) must be within relative RMS 2e-3 of the oracle's (the
pages report ~1e-3 per expert against fp64 for their own CPU and fused GPU
kernels: page "0xSero/glm53-flash-offload", paragraph "Reference: a
teacher-forced panel"), and so must every token's combined output.
"""
import numpy as np
import pytest
import torch

import bit_moe_expert_router_amd as moe

import oracle
import synth
from synth.device import DeviceLayer, x_device
from tests.gpu_util import HostExperts, make_layer_api, rel_err, run_gpu, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
W_TOL = 2e-7  # routing weights: fp64 values rounded to fp32

_layers = {}


def layer_for(name, device, slots=None):
    key = (name, None if slots is None else tuple(slots))
    if key not in _layers:
        cfg = synth.CONFIGS[name]
        _layers[key] = DeviceLayer.generate(cfg, 0, device, slots=slots)
    return _layers[key]


def check_routing(cfg, xh, res):
    ids, w, gap, _ = oracle.route(xh, synth.router_f32(cfg), synth.zipf_bias(cfg), cfg.top_k)
    assert np.array_equal(res["ids"], ids), "routing ids differ"
    assert np.all(np.abs(res["w"] - w) <= W_TOL * np.maximum(w, 1e-30) + 1e-12)
    off, sp, pp = oracle.permute(ids, cfg.n_experts)
    assert np.array_equal(res["offsets"], off)
    assert np.array_equal(res["sorted"], sp)
    assert np.array_equal(res["pos"], pp)
    return ids, w


def test_device_fill_matches_host_generator(gpu):
    for name, experts in (("c1", range(16)), ("c3", (0, 17, 287))):
        say(f"[fill] {name}")
        cfg = synth.CONFIGS[name]
        dl = layer_for(name, gpu)
        for e in experts:
            assert np.array_equal(dl.expert_host(e), synth.expert_blob(cfg, 0, e)), (name, e)
        if cfg.shared_inter:
            host = synth.shared_weights(cfg)
            for dev_t, h in zip(dl.shared, host):
                assert np.array_equal(dev_t.cpu().numpy().view(np.uint16), h)


ROUTE_CASES = [("c1", 4), ("c1", 1), ("c1", 3), ("c1", 16), ("c1", 37), ("c2", 1), ("c2", 2),
               ("c2", 3), ("c2", 4), ("c2", 5),
               ("c3", 8), ("c3", 64), ("c3", 65), ("c3", 300), ("c5", 8192)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_routing_bit_exact(gpu, name, T):
    say(f"[route] {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    r = ml.route(xd, dl.router, dl.bias)
    torch.cuda.synchronize()
    res = dict(ids=r.topk_ids.cpu().numpy(), w=r.topk_w.cpu().numpy(),
               offsets=r.expert_offsets.cpu().numpy(), sorted=r.sorted_pairs.cpu().numpy(),
               pos=r.pair_pos.cpu().numpy())
    check_routing(cfg, xh, res)
    ml.close()


# decode batches run the GEMV kernels; T > 64 the matrix-core (prefill) kernels:
# the 4-bit/G32/fp16-scale shape at T = 300 and the GLM shape just past the switch.
# c3 at T = 16 and 64 gives the hottest experts more tokens than one chunk of the
# GEMVs takes (8 for gate/up, 4 for down), so their later chunks run.
FFN_CASES = [("c1", 4), ("c1", 1), ("c1", 13), ("c2", 1), ("c2", 3), ("c3", 1), ("c3", 2),
             ("c3", 8), ("c3", 9), ("c3", 16), ("c3", 64), ("c1", 300), ("c2", 65),
             ("q2", 1), ("q2", 2), ("q2", 8), ("q2", 65), ("q4", 1), ("q4", 2), ("q4", 8),
             ("q4", 65)]


def check_all_pairs(cfg, xh, res, ids, w, he, label):
    """every pair's expert output and every token's combined output against the
    oracle; returns the worst pair error"""
    T, K = ids.shape
    refs = he.ffn_pairs(xh, ids, range(T * K))
    worst = 0.0
    for p in range(T * K):
        r = rel_err(res["pair_out"][p], refs[p])
        worst = max(worst, r)
        assert r <= TOL, (label, p, int(ids.reshape(-1)[p]), r)
    sh = he.shared()
    if T <= 9:  # the oracle's whole layer, an independent path through the combine
        tabs = [[he.blobs(e)[m] for e in range(cfg.n_experts)] for m in range(3)]
        out, _ = oracle.moe_layer(xh, ids, w, *tabs, cfg.inter, cfg.bits, cfg.group,
                                  cfg.scale_f16, sh)
    else:  # sum_k w y(t,k) (k ascending) + shared, from the oracle's pair outputs
        out = np.zeros((T, cfg.hidden))
        for t in range(T):
            for k in range(K):
                out[t] += np.float64(w[t, k]) * refs[t * K + k]
            if sh is not None:
                out[t] += oracle.shared_ffn(synth.bf16_to_f32(xh[t]).astype(np.float64), *sh)
    for t in range(T):
        assert rel_err(res["out"][t], out[t]) <= TOL, (label, t)
    return worst


@pytest.mark.parametrize("name,T", FFN_CASES)
def test_expert_outputs_all_pairs(gpu, name, T):
    say(f"[ffn] {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    res = run_gpu(cfg, dl, xd)
    ids, w = check_routing(cfg, xh, res)
    counts = np.diff(res["offsets"])
    worst = check_all_pairs(cfg, xh, res, ids, w, HostExperts(cfg), f"{name} T={T}")
    say(f"[ffn] {name} T={T} worst pair rel err {worst:.3e}, most pairs per expert {counts.max()}")


@pytest.mark.parametrize("T,n_hot", [(9, 9), (40, 40), (64, 64)])
def test_decode_long_expert_segments(gpu, T, n_hot):
    """caller-supplied routing in which one expert takes every token (n_hot pairs)
    and a second one every other token: the GEMVs' later token chunks (gate/up
    takes 8 positions per chunk, down 4) all run against the oracle"""
    say(f"[ffn] long segments c3 T={T}")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    a = run_gpu(cfg, dl, xd, ml=ml)
    ids, w = a["ids"].copy(), a["w"].copy()
    hot, second = 17, 251
    for t in range(T):
        row = [e for e in ids[t] if e not in (hot, second)]
        row = [hot] + ([second] if t % 2 == 0 else []) + row
        ids[t] = np.array(row[:cfg.top_k], dtype=np.int32)
    r = _caller_routing(ml, ids, w, cfg.n_experts, gpu)
    b = run_gpu(cfg, dl, xd, ml=ml, routing=r)
    counts = np.diff(b["offsets"])
    assert counts[hot] == n_hot and counts[second] == (T + 1) // 2
    worst = check_all_pairs(cfg, xh, b, ids, w, HostExperts(cfg), f"long T={T}")
    say(f"[ffn] long segments T={T}: worst pair rel err {worst:.3e}")
    ml.close()


def _prefill_check(gpu, cfg, label):
    """8,192-token chunk: routing of every token bit-exact; every pair of one full
    128-position tile of the hottest expert and of the median expert, both ends of
    the coldest expert, random pairs, and the combined output of 16 tokens"""
    T = cfg.tokens
    dl = layer_for("c5", gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    r = ml.route(xd, dl.router, dl.bias if cfg.zipf else None)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    pair_out = torch.empty((T * cfg.top_k, cfg.hidden), dtype=torch.float32, device=gpu)
    ml.forward(0, xd, r, out, pair_out)
    torch.cuda.synchronize()
    res = dict(ids=r.topk_ids.cpu().numpy(), w=r.topk_w.cpu().numpy(),
               offsets=r.expert_offsets.cpu().numpy(), sorted=r.sorted_pairs.cpu().numpy(),
               pos=r.pair_pos.cpu().numpy())
    ids, w = check_routing(cfg, xh, res)
    off, sp = res["offsets"], res["sorted"]
    counts = np.diff(off)
    order = np.argsort(counts, kind="stable")
    hot = int(order[-1])
    live = order[counts[order] > 0]
    med = int(live[len(live) // 2])
    cold = int(live[0])
    pairs = set(sp[off[hot]:off[hot] + min(128, counts[hot])].tolist())
    pairs |= set(sp[off[med]:off[med] + min(128, counts[med])].tolist())
    pairs |= {int(sp[off[cold]]), int(sp[off[cold + 1] - 1])}
    rng = np.random.default_rng(0)
    pairs |= set(rng.integers(0, T * cfg.top_k, size=32).tolist())
    toks = sorted(set(rng.integers(0, T, size=16).tolist()) | {0, T - 1})
    pairs |= {t * cfg.top_k + k for t in toks for k in range(cfg.top_k)}
    he = HostExperts(cfg)
    refs = he.ffn_pairs(xh, ids, sorted(pairs))
    po = pair_out.cpu().numpy()
    worst = 0.0
    for p, y in refs.items():
        e = int(ids.reshape(-1)[p])
        err = rel_err(po[p], y)
        worst = max(worst, err)
        assert err <= TOL, (label, p, e, err)
    o = out.cpu().numpy()
    for t in toks:
        ref = sum(np.float64(w[t, k]) * refs[t * cfg.top_k + k] for k in range(cfg.top_k))
        assert rel_err(o[t], ref) <= TOL, (label, t)
    say(f"[prefill] {label}: hot expert {hot} {counts[hot]} pairs, median {med} {counts[med]}, "
        f"{len(refs)} pairs checked, worst {worst:.3e}")
    ml.close()


@pytest.mark.parametrize("zipf", [True, False], ids=["zipf", "uniform"])
def test_prefill_chunk(gpu, zipf):
    cfg = synth.CONFIGS["c5"].with_(zipf=zipf)
    say(f"[prefill] c5 T={cfg.tokens} {'zipf' if zipf else 'uniform'}")
    _prefill_check(gpu, cfg, "zipf" if zipf else "uniform")


def test_prefill_ragged_tiles(gpu):
    """300 tokens through the matrix-core kernels at the GLM shape with the shared
    expert: every pair of the hottest expert (several 128-row tiles, the last one
    ragged), every pair of experts with a single pair, random pairs, and the
    combined output (routed + shared) of sampled tokens."""
    name, T = "c3", 300
    say(f"[prefill] {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    res = run_gpu(cfg, dl, xd)
    ids, w = check_routing(cfg, xh, res)
    off, sp = res["offsets"], res["sorted"]
    counts = np.diff(off)
    hot = int(np.argmax(counts))
    assert counts[hot] > 128 and counts[hot] % 128 != 0, counts[hot]
    pairs = set(sp[off[hot]:off[hot + 1]].tolist())
    singles = np.nonzero(counts == 1)[0][:2]
    pairs |= {int(sp[off[e]]) for e in singles}
    rng = np.random.default_rng(1)
    pairs |= set(rng.integers(0, T * cfg.top_k, size=32).tolist())
    toks = rng.integers(0, T, size=3).tolist()
    pairs |= {t * cfg.top_k + k for t in toks for k in range(cfg.top_k)}
    he = HostExperts(cfg)
    refs = he.ffn_pairs(xh, ids, sorted(pairs))
    worst = 0.0
    for p, y in refs.items():
        r = rel_err(res["pair_out"][p], y)
        worst = max(worst, r)
        assert r <= TOL, (p, int(ids.reshape(-1)[p]), r)
    sh = he.shared()
    for t in toks:
        ref = sum(np.float64(w[t, k]) * refs[t * cfg.top_k + k] for k in range(cfg.top_k))
        ref = ref + oracle.shared_ffn(synth.bf16_to_f32(xh[t]).astype(np.float64), *sh)
        assert rel_err(res["out"][t], ref) <= TOL, t
    say(f"[prefill] hot expert {hot}: {counts[hot]} pairs; worst pair rel err {worst:.3e}")


# ------------------------------------------------------------------ invariants
def test_run_twice_bit_identical(gpu):
    say("[inv] run twice")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    _, xd = x_device(cfg, gpu)
    a = run_gpu(cfg, dl, xd)
    b = run_gpu(cfg, dl, xd, ml=a["ml"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["pair_out"], b["pair_out"])


def test_token_reorder_permutes_outputs(gpu):
    say("[inv] reorder")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    xh, xd = x_device(cfg, gpu)
    a = run_gpu(cfg, dl, xd)
    perm = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    b = run_gpu(cfg, dl, xd[torch.from_numpy(perm).to(gpu)].contiguous())
    assert np.array_equal(b["ids"], a["ids"][perm])
    assert np.array_equal(b["out"], a["out"][perm])


def test_remap_bit_identical(gpu):
    """the same logical experts at other physical slots give bit-identical results"""
    say("[inv] remap")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    other = synth.permutation(cfg.n_experts, 1234, 0, synth.SYN_SLOT_PERM)
    assert not np.array_equal(other, dl.slots)
    dl2 = layer_for("c3", gpu, slots=other)
    _, xd = x_device(cfg, gpu)
    a = run_gpu(cfg, dl, xd)
    b = run_gpu(cfg, dl2, xd)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["pair_out"], b["pair_out"])
    # remapping one context's table in place of the old one does the same
    ml = a["ml"]
    ml.set_table(0, dl2.refs)
    c = run_gpu(cfg, dl2, xd, ml=ml)
    assert np.array_equal(a["out"], c["out"])


def _caller_routing(ml, ids, w, E, device):
    from bit_moe_expert_router_amd import RoutingBuffers
    off, sp, pp = oracle.permute(ids, E)
    T, K = ids.shape
    sp_full = np.zeros(T * K, dtype=np.int32)
    sp_full[:sp.size] = sp
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(device)
    return RoutingBuffers(t(ids, np.int32), t(w, np.float32), t(off, np.int32),
                          t(sp_full, np.int32), t(pp, np.int32))


def test_zero_weight_pair_equals_dropped_pair(gpu):
    say("[inv] zero weight")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    xh, xd = x_device(cfg, gpu)
    a = run_gpu(cfg, dl, xd)
    ids, w = a["ids"].copy(), a["w"].copy()
    w[3, 5] = 0.0
    r0 = _caller_routing(a["ml"], ids, w, cfg.n_experts, gpu)
    b = run_gpu(cfg, dl, xd, ml=a["ml"], routing=r0)
    ids_d = ids.copy()
    ids_d[3, 5] = -1
    r1 = _caller_routing(a["ml"], ids_d, w, cfg.n_experts, gpu)
    c = run_gpu(cfg, dl, xd, ml=a["ml"], routing=r1)
    assert np.array_equal(b["out"], c["out"])
    # and the dropped pair matches the oracle's treatment of an id outside [0, E)
    he = HostExperts(cfg)
    tabs = [[he.blobs(e)[m] for e in range(cfg.n_experts)] for m in range(3)]
    ref, _ = oracle.moe_layer(xh, ids_d, w.astype(np.float64), *tabs, cfg.inter, cfg.bits,
                              cfg.group, cfg.scale_f16, he.shared())
    assert rel_err(c["out"][3], ref[3]) <= TOL


@pytest.mark.parametrize("name,T", [("c2", 1), ("c3", 1), ("c3", 2)])
def test_small_batch_all_pairs_dropped(gpu, name, T):
    """one/two-token batches with every pair left out: no expert runs, and each
    token's output is the shared expert's alone (zero without one)"""
    say(f"[inv] all dropped {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ids = np.full((T, cfg.top_k), -1, dtype=np.int32)
    w = np.full((T, cfg.top_k), 1.0 / cfg.top_k, dtype=np.float32)
    ml = make_layer_api(cfg, dl, T)
    res = run_gpu(cfg, dl, xd, ml=ml, routing=_caller_routing(ml, ids, w, cfg.n_experts, gpu))
    he = HostExperts(cfg)
    dummy = [[np.zeros(16, np.uint8)] * cfg.n_experts for _ in range(3)]
    ref, _ = oracle.moe_layer(xh, ids, w.astype(np.float64), *dummy, cfg.inter, cfg.bits,
                              cfg.group, cfg.scale_f16, he.shared())
    for t in range(T):
        if he.shared() is None:
            assert not np.any(res["out"][t]), t
        else:
            assert rel_err(res["out"][t], ref[t]) <= TOL, t
    ml.close()


@pytest.mark.parametrize("name", ["c2", "c3"])
@pytest.mark.parametrize("T", [1, 2])
def test_small_batch_repeated_expert(gpu, name, T):
    """caller-supplied routing that lists one expert twice per token: at two
    tokens the expert owns four positions, more than a single pass of the
    one/two-token kernels takes, so their later passes run; at one token it owns
    two, and every expert above it sits one position later than its rank, so the
    down kernel's early h requests (position a for the a-th expert) miss there
    and are made again; every pair and the combined output against the oracle"""
    say(f"[ffn] repeated expert {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    a = run_gpu(cfg, dl, xd, ml=ml)
    ids, w = a["ids"].copy(), a["w"].copy()
    e = int(ids[0, 0])
    ids[0, 1] = e
    if T == 2:
        ids[1, 0] = e
        ids[1, 1] = e
    r = _caller_routing(ml, ids, w, cfg.n_experts, gpu)
    b = run_gpu(cfg, dl, xd, ml=ml, routing=r)
    assert np.diff(b["offsets"])[e] == 2 * T
    he = HostExperts(cfg)
    for t in range(T):
        for k in range(cfg.top_k):
            ref = he.ffn(xh[t], int(ids[t, k]))
            assert rel_err(b["pair_out"][t * cfg.top_k + k], ref) <= TOL, (t, k)
    tabs = [[he.blobs(q)[m] for q in range(cfg.n_experts)] for m in range(3)]
    out_ref, _ = oracle.moe_layer(xh, ids, w.astype(np.float64), *tabs, cfg.inter, cfg.bits,
                                  cfg.group, cfg.scale_f16, he.shared())
    for t in range(T):
        assert rel_err(b["out"][t], out_ref[t]) <= TOL, t
    ml.close()


def test_counters_left_zero(gpu):
    """the workspace's cross-block counters are zero again after every call"""
    say("[inv] counters")
    cfg = synth.CONFIGS["c3"]
    dl = layer_for("c3", gpu)
    ml = make_layer_api(cfg, dl, 64)
    for T in (1, 2, 5, 8, 64):
        _, xd = x_device(cfg, gpu, tokens=T)
        for _ in range(2):
            run_gpu(cfg, dl, xd, ml=ml)
        ctr = ml.ws[:moe.MOE_WS_COUNTER_BYTES].view(torch.int32)
        assert int(torch.count_nonzero(ctr)) == 0, T
    ml.close()


# ------------------------------------------------------------------ status codes
def test_status_codes(gpu):
    import bit_moe_expert_router_amd as m
    say("[abi] status codes")
    cfg = synth.CONFIGS["c1"]
    dl = layer_for("c1", gpu)
    xh, xd = x_device(cfg, gpu, tokens=4)
    ml = m.MoELayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits, cfg.group,
                    cfg.scale_f16, 0, 4, 1, gpu)
    r = ml.routing(4)
    out = torch.empty((4, cfg.hidden), dtype=torch.float32, device=gpu)
    with pytest.raises(m.MoEError) as ei:  # table never set
        ml.forward(0, xd, r, out)
    assert ei.value.status == m.MOE_E_STATE
    ml.set_table(0, dl.refs)
    x5 = torch.zeros((5, cfg.hidden), dtype=torch.int16, device=gpu)
    with pytest.raises(m.MoEError) as ei:  # T above max_tokens
        ml.route(x5, dl.router)
    assert ei.value.status == m.MOE_E_ARG
    small = torch.zeros(1024, dtype=torch.uint8, device=gpu)
    with pytest.raises(m.MoEError) as ei:  # workspace too small
        m.moe_route(ml.ctx, xd, 4, dl.router, None, r.topk_ids, r.topk_w, r.expert_offsets,
                    r.sorted_pairs, r.pair_pos, small)
    assert ei.value.status == m.MOE_E_ARG
    with pytest.raises(m.MoEError) as ei:  # misaligned activations
        m.moe_route(ml.ctx, xd.data_ptr() + 2, 3, dl.router, None, r.topk_ids, r.topk_w,
                    r.expert_offsets, r.sorted_pairs, r.pair_pos, ml.ws)
    assert ei.value.status == m.MOE_E_ARG
    bad = list(dl.refs)
    bad[3] = (bad[3][0] + 16, bad[3][1], bad[3][2])
    with pytest.raises(m.MoEError) as ei:  # blob not 256-byte aligned
        ml.set_table(0, bad)
    assert ei.value.status == m.MOE_E_ARG
    # T = 0 is a no-op
    m.moe_route(ml.ctx, xd, 0, dl.router, None, r.topk_ids, r.topk_w, r.expert_offsets,
                r.sorted_pairs, r.pair_pos, ml.ws)
    ml.close()


# ------------------------------------------------------------------ graph replay
@pytest.mark.parametrize("name,T", [("c2", 1), ("c3", 8), ("c3", 5)])
def test_graph_replay_matches_eager(gpu, name, T):
    """route + forward captured in one HIP graph: every replay (with eager work of
    other batch sizes in between, which moves the workspace counters and
    buffers) equals the eager result bit for bit"""
    say(f"[graph] {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, 16)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    r = ml.route(xd, dl.router, dl.bias)
    ml.forward(0, xd, r, out)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r = ml.route(xd, dl.router, dl.bias)
        ml.forward(0, xd, r, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r = ml.route(xd, dl.router, dl.bias)
        ml.forward(0, xd, r, out)
    _, x_other = x_device(cfg, gpu, tokens=16)
    other = torch.empty((16, cfg.hidden), dtype=torch.float32, device=gpu)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        ro = ml.route(x_other, dl.router, dl.bias)  # eager work between replays
        ml.forward(0, x_other, ro, other)
        torch.cuda.synchronize()
    ml.close()


def _out_only(ml, xd, r, H):
    out = torch.empty((xd.shape[0], H), dtype=torch.float32, device=xd.device)
    ml.forward(0, xd, r, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


COMBINE_CASES = [("c1", 4), ("c2", 1), ("c2", 2), ("c2", 3), ("c3", 2), ("c3", 4), ("c3", 8),
                 ("c3", 9), ("q2", 8), ("q4", 5)]


@pytest.mark.parametrize("name,T", COMBINE_CASES)
def test_combined_output_without_pair_outputs(gpu, name, T):
    """a call that asks for the combined output only (decode batches of up to
    eight tokens then combine inside the down kernel): every token against the
    oracle's layer, against the same call with pair outputs (a different
    summation of the same terms), and bit-identical on a second run"""
    say(f"[ffn] out only {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    a = run_gpu(cfg, dl, xd, ml=ml)
    r = _caller_routing(ml, a["ids"], a["w"], cfg.n_experts, gpu)
    b = _out_only(ml, xd, r, cfg.hidden)
    c = _out_only(ml, xd, r, cfg.hidden)
    assert np.array_equal(b, c)
    he = HostExperts(cfg)
    tabs = [[he.blobs(q)[m] for q in range(cfg.n_experts)] for m in range(3)]
    ref, _ = oracle.moe_layer(xh, a["ids"], a["w"].astype(np.float64), *tabs, cfg.inter,
                              cfg.bits, cfg.group, cfg.scale_f16, he.shared())
    for t in range(T):
        assert rel_err(b[t], ref[t]) <= TOL, t
        assert rel_err(b[t], a["out"][t].astype(np.float64)) <= 1e-5, t
    ml.close()


@pytest.mark.parametrize("name,T", [("c3", 4), ("c2", 8)])
def test_combined_output_dropped_pairs(gpu, name, T):
    """combined output only, with caller routing in which token 1 has no valid
    pair (its output is the shared expert's alone) and token 2 one pair left out"""
    say(f"[ffn] out only, dropped pairs {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    a = run_gpu(cfg, dl, xd, ml=ml)
    ids, w = a["ids"].copy(), a["w"].copy()
    ids[1, :] = -1
    ids[2, 3] = cfg.n_experts
    b = _out_only(ml, xd, _caller_routing(ml, ids, w, cfg.n_experts, gpu), cfg.hidden)
    assert ml.error_word() == 0
    he = HostExperts(cfg)
    tabs = [[he.blobs(q)[m] for q in range(cfg.n_experts)] for m in range(3)]
    ref, _ = oracle.moe_layer(xh, ids, w.astype(np.float64), *tabs, cfg.inter, cfg.bits,
                              cfg.group, cfg.scale_f16, he.shared())
    for t in range(T):
        if t == 1 and he.shared() is None:
            assert not np.any(b[t])
        else:
            assert rel_err(b[t], ref[t]) <= TOL, t
    ctr = ml.ws[:moe.MOE_WS_COUNTER_BYTES].view(torch.int32)
    assert int(torch.count_nonzero(ctr)) == 0
    ml.close()


LAYER_CASES = [("c1", 1), ("c1", 2), ("c1", 4), ("c1", 8), ("c2", 1), ("c2", 2), ("c2", 3),
               ("c3", 1), ("c3", 2), ("c3", 8), ("c3", 9), ("q2", 1), ("q2", 8), ("q4", 2),
               ("q4", 5), ("c2", 65)]


@pytest.mark.parametrize("name,T", LAYER_CASES)
def test_layer_forward_equals_route_then_forward(gpu, name, T):
    """moe_layer_forward (routing and experts in one call; at one and two tokens
    the routing kernel hands the expert entries to the expert kernels, at three to
    eight it also does the decode plan: the active list and the codec's offset
    sums) gives the routing and the outputs of moe_route followed by moe_forward,
    bit for bit, with and without pair outputs"""
    say(f"[ffn] layer call {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = layer_for(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    a = run_gpu(cfg, dl, xd, ml=ml)
    for with_po in (True, False):
        out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
        po = (torch.empty((T * cfg.top_k, cfg.hidden), dtype=torch.float32, device=gpu)
              if with_po else None)
        r = ml.layer_forward(0, xd, dl.router, dl.bias, out, po)
        torch.cuda.synchronize()
        assert np.array_equal(r.topk_ids.cpu().numpy(), a["ids"])
        assert np.array_equal(r.topk_w.cpu().numpy(), a["w"])
        assert np.array_equal(r.expert_offsets.cpu().numpy(), a["offsets"])
        assert np.array_equal(r.sorted_pairs.cpu().numpy(), a["sorted"])
        assert np.array_equal(r.pair_pos.cpu().numpy(), a["pos"])
        assert np.array_equal(out.cpu().numpy(), a["out"]), with_po
        if with_po:
            assert np.array_equal(po.cpu().numpy(), a["pair_out"])
    assert ml.error_word() == 0
    ctr = ml.ws[:moe.MOE_WS_COUNTER_BYTES].view(torch.int32)
    assert int(torch.count_nonzero(ctr)) == 0
    ml.close()
