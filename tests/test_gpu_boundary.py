"""The boundary's device-side contract: caller-supplied routing checked on the
device (error word, outputs untouched), set_expert_table that neither waits nor
breaks graph capture, and in-place device rewrites of a layer's table.

The inconsistent routings below keep every value inside the buffers' extents
(positions and pair ids within [0, T*K], the ids buffer padded by one row), so
that even a kernel without the checks could not read outside them."""
import numpy as np
import pytest
import torch

import bit_moe_expert_router_amd as moe

import oracle
import synth
from synth.device import DeviceLayer, x_device
from tests.gpu_util import make_layer_api, say

pytestmark = pytest.mark.gpu

SENT = 0x7FC0BEEF  # a NaN bit pattern the kernels never produce

_layers = {}


def _layer(name, dev, slots=None):
    key = (name, None if slots is None else tuple(slots))
    if key not in _layers:
        _layers[key] = DeviceLayer.generate(synth.CONFIGS[name], 0, dev, slots=slots)
    return _layers[key]


def _routing(ml, ids, w, off, sp, dev):
    """RoutingBuffers over caller arrays; the ids buffer has one spare row"""
    from bit_moe_expert_router_amd import RoutingBuffers
    T, K = ids.shape
    ids_pad = np.concatenate([ids, np.zeros((1, K), np.int32)]).astype(np.int32)
    sp_full = np.zeros(T * K, np.int32)
    sp_full[:len(sp)] = sp
    d = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).to(dev)
    ids_d = d(ids_pad, np.int32)
    pp = np.zeros(T * K, np.int32)
    return RoutingBuffers(ids_d[:T], d(w, np.float32), d(off, np.int32), d(sp_full, np.int32),
                          d(pp, np.int32))


def _forward(ml, x, r, T, H, K, with_pair_out):
    """outputs with one spare row each (untouched by any call), filled with SENT"""
    out = torch.empty((T + 1, H), dtype=torch.float32, device=x.device)
    out.view(torch.int32).fill_(SENT)
    po = None
    if with_pair_out:
        po = torch.empty(((T + 1) * K, H), dtype=torch.float32, device=x.device)
        po.view(torch.int32).fill_(SENT)
    ml.forward(0, x[:T], r, out[:T], None if po is None else po[:T * K])
    torch.cuda.synchronize()
    assert torch.all(out[T].view(torch.int32) == SENT)
    if po is not None:
        assert torch.all(po[T * K:].view(torch.int32) == SENT)
    return out[:T], None if po is None else po[:T * K]


def _corruptions(ids, off, sp, E):
    """(name, ids, offsets, sorted_pairs) variants that are each inconsistent"""
    T, K = ids.shape
    P = T * K
    counts = np.diff(off)
    act = np.nonzero(counts > 0)[0]
    out = []
    # two pairs of different experts swapped in the grouping
    s = sp.copy()
    i, j = off[act[0]], off[act[-1]]
    s[i], s[j] = s[j], s[i]
    out.append(("swap", ids, off, s))
    # a pair listed twice within its expert, another one missing
    big = act[np.argmax(counts[act])]
    if counts[big] >= 2:
        s = sp.copy()
        s[off[big] + 1] = s[off[big]]
        out.append(("duplicate", ids, off, s))
    # the grouping one pair short of the valid pairs
    o = off.copy()
    o[-1] -= 1
    out.append(("short", ids, o, sp))
    # offsets that decrease (values kept inside [0, P])
    o = off.copy()
    k = act[0]
    o[k + 1] = max(o[k] - 1, 0)
    if o[k + 1] < o[k]:
        out.append(("decreasing", ids, o, sp))
    # a pair id one past the last pair
    s = sp.copy()
    s[off[act[-1]]] = P
    out.append(("pair range", ids, off, s))
    # an id changed without regrouping
    i2 = ids.copy()
    t0, k0 = divmod(int(sp[0]), K)
    i2[t0, k0] = (i2[t0, k0] + 1) % E
    out.append(("id changed", i2, off, sp))
    return out


CASES = [("c1", 4), ("c2", 1), ("c3", 2), ("c3", 8), ("c3", 64), ("c3", 300)]


@pytest.mark.parametrize("name,T", CASES)
def test_inconsistent_routing_sets_error_word(gpu, name, T):
    cfg = synth.CONFIGS[name]
    say(f"[boundary] bad routing {name} T={T}")
    dl = _layer(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T + 1)  # a spare token row
    xh = xh[:T]
    ml = make_layer_api(cfg, dl, T)
    H, K, E = cfg.hidden, cfg.top_k, cfg.n_experts
    ids, w, _, _ = oracle.route(xh, synth.router_f32(cfg), synth.zipf_bias(cfg), K)
    off, sp, _ = oracle.permute(ids, E)
    good = _routing(ml, ids, w, off, sp, gpu)
    ref_out, ref_po = _forward(ml, xd, good, T, H, K, True)
    assert ml.error_word() == 0
    assert not torch.any(ref_out.view(torch.int32) == SENT)
    for label, i2, o2, s2 in _corruptions(ids, off, sp, E):
        for with_po in (True, False):
            r = _routing(ml, i2, w, o2, s2, gpu)
            out, po = _forward(ml, xd, r, T, H, K, with_po)
            assert ml.error_word() & 1, (label, with_po)
            assert torch.all(out.view(torch.int32) == SENT), (label, "out written")
            if po is not None:
                assert torch.all(po.view(torch.int32) == SENT), (label, "pair_out written")
            ml.clear_error()
        # a consistent call right after is unaffected, and leaves the word clear
        out, po = _forward(ml, xd, good, T, H, K, True)
        assert torch.equal(out, ref_out) and torch.equal(po, ref_po), label
        assert ml.error_word() == 0, label
    ctr = ml.ws[:moe.MOE_WS_COUNTER_BYTES].view(torch.int32)
    assert int(torch.count_nonzero(ctr)) == 0
    ml.close()


def test_set_table_does_not_wait_and_captures(gpu):
    """set_expert_table inside a captured graph: the replays use the entries as
    they were at capture (the host array is overwritten right after the call),
    and the graph's own set overrides an eager set made between replays"""
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c3"]
    say("[boundary] set_expert_table under capture")
    dl = _layer("c3", gpu)
    T = 8
    _, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    r = ml.route(xd, dl.router, dl.bias)
    ml.forward(0, xd, r, out)
    torch.cuda.synchronize()
    ref_a = out.clone()
    ids = r.topk_ids.cpu().numpy()
    e0, e1 = int(ids[0, 0]), int(ids[0, 1])
    refs_b = list(dl.refs)
    refs_b[e0], refs_b[e1] = refs_b[e1], refs_b[e0]  # two experts' bytes swapped
    ml.set_table(0, refs_b)
    ml.forward(0, xd, r, out)
    torch.cuda.synchronize()
    ref_b = out.clone()
    assert not torch.equal(ref_a, ref_b)
    ml.set_table(0, dl.refs)
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        ml.set_table(0, dl.refs)
        r = ml.route(xd, dl.router, dl.bias)
        ml.forward(0, xd, r, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_a)
    g = torch.cuda.CUDAGraph()
    arr = (m.moe_expert_ref * cfg.n_experts)(*[m.moe_expert_ref(*t) for t in refs_b])
    with torch.cuda.graph(g):
        st = m.lib.set_expert_table(ml.ctx, 0, arr, torch.cuda.current_stream().cuda_stream)
        assert st == m.MOE_OK
        for i in range(cfg.n_experts):  # the host array is reused at once (table A again:
            arr[i] = m.moe_expert_ref(*dl.refs[i])  # valid addresses, other results)
        r = ml.route(xd, dl.router, dl.bias)
        ml.forward(0, xd, r, out)
    for rep in range(3):
        ml.set_table(0, dl.refs)  # eager: back to table A
        ml.forward(0, xd, r, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a), rep
        out.zero_()
        g.replay()  # sets table B itself
        torch.cuda.synchronize()
        assert torch.equal(out, ref_b), rep
    ml.close()


class _DevView:
    """a device buffer at a raw address, as a torch tensor"""

    def __init__(self, ptr, nbytes):
        self.__cuda_array_interface__ = {"shape": (nbytes // 8,), "typestr": "<i8",
                                         "data": (ptr, False), "version": 2}


def test_table_rewritten_on_device(gpu):
    """a table rewritten in place through moe_expert_table_device (a device copy
    stream-ordered before the forward) gives bit-identical outputs to setting it
    from the host"""
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c3"]
    say("[boundary] device-side table rewrite")
    dl = _layer("c3", gpu)
    other = synth.permutation(cfg.n_experts, 99, 0, synth.SYN_SLOT_PERM)
    dl2 = _layer("c3", gpu, slots=other)
    T = 5
    _, xd = x_device(cfg, gpu, tokens=T)
    ml = make_layer_api(cfg, dl, T)
    addr = m.moe_expert_table_device(ml.ctx, 0)
    assert addr and m.moe_expert_table_device(ml.ctx, 1) == 0
    tab = torch.as_tensor(_DevView(addr, 24 * cfg.n_experts), device=gpu)
    assert tab.data_ptr() == addr
    assert torch.equal(tab.cpu(), torch.tensor(dl.refs, dtype=torch.int64).reshape(-1))
    out_a = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    r = ml.route(xd, dl.router, dl.bias)
    ml.forward(0, xd, r, out_a)
    new = torch.tensor(dl2.refs, dtype=torch.int64, device=gpu).reshape(-1)
    tab.copy_(new)  # device-to-device, on the current stream
    out_b = torch.empty_like(out_a)
    ml.forward(0, xd, r, out_b)
    torch.cuda.synchronize()
    assert torch.equal(tab.cpu(), new.cpu())
    assert torch.equal(out_a, out_b)
    # a slot pointing at another logical expert's bytes changes that expert's output
    swap = new.clone().reshape(cfg.n_experts, 3)
    ids = r.topk_ids.cpu().numpy()
    e0, e1 = int(ids[0, 0]), int(ids[0, 1])
    swap[[e0, e1]] = swap[[e1, e0]]
    tab.copy_(swap.reshape(-1))
    out_c = torch.empty_like(out_a)
    ml.forward(0, xd, r, out_c)
    torch.cuda.synchronize()
    assert not torch.equal(out_c[0], out_a[0])
    ml.close()


def test_stream_read_probe(gpu):
    """the streaming-read probe (a measurement aid) reads without writing, and
    refuses sizes that are not whole 16-byte vectors"""
    import bit_moe_expert_router_amd as m
    say("[boundary] stream-read probe")
    src = torch.arange(1 << 18, dtype=torch.int32, device=gpu)  # 1 MiB
    sink = torch.zeros(4096 * 256, dtype=torch.int32, device=gpu)
    m.moe_stream_read(src, src.numel() * 4, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0
    with pytest.raises(m.MoEError) as ei:
        m.moe_stream_read(src, 1000, sink)
    assert ei.value.status == m.MOE_E_ARG


def test_prefill_range_flag(gpu):
    """The matrix-core path (T > 64) holds expanded weights q*s and h = silu(g)*u
    in fp16: it sets MOE_ERR_RANGE when a value leaves fp16's exact range.
    Ordinary inputs leave the error word clear; activations scaled by 2^9 make
    |h| exceed 65504; one group scale of 2^14 in a used expert makes q*s inexact
    (restored afterwards).  No value here can fault: they are only numbers."""
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c3"]
    T = 100
    say("[boundary] prefill fp16 range flag")
    dl = _layer("c3", gpu)
    ml = make_layer_api(cfg, dl, T)
    xh, xd = x_device(cfg, gpu, tokens=T)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)

    def run(x):
        ml.clear_error()
        r = ml.route(x, dl.router, dl.bias)
        ml.forward(0, x, r, out)
        torch.cuda.synchronize()
        return ml.error_word(), r

    e0, r = run(xd)
    assert e0 == 0, e0
    big = (xd.view(torch.bfloat16).float() * 512.0).to(torch.bfloat16).view(torch.int16)
    e1, _ = run(big)
    assert e1 & m.MOE_ERR_RANGE, e1
    # one scale of the hottest expert's gate matrix set to 2^14 (bf16 0x4680)
    off = r.expert_offsets.cpu().numpy()
    hot = int(np.argmax(np.diff(off)))
    lay = synth.matrix_layout(cfg.inter, cfg.hidden, cfg.bits, cfg.group)
    addr = dl.refs[hot][0] + lay.scales_off
    a = addr - dl.arena.data_ptr()
    saved = dl.arena[a:a + 2].clone()
    dl.arena[a:a + 2] = torch.tensor([0x80, 0x46], dtype=torch.uint8, device=gpu)
    try:
        e2, _ = run(xd)
    finally:
        dl.arena[a:a + 2] = saved
    torch.cuda.synchronize()
    assert e2 & m.MOE_ERR_RANGE, e2
    e3, _ = run(xd)
    assert e3 == 0, e3
    ml.close()


def test_profile_stats_match_raw_reads(gpu):
    """per-kernel timing: the same steps read once as totals and once as
    statistics give the same kernels and launch counts; medians and typical
    means are positive, and the typical mean (launches within twice the median)
    is at most twice the median"""
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c1"]
    say("[boundary] profile statistics")
    dl = _layer("c1", gpu)
    T, steps = 4, 6
    ml = make_layer_api(cfg, dl, T)
    xh, xd = x_device(cfg, gpu, tokens=T)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)

    def run():
        for _ in range(steps):
            r = ml.route(xd, dl.router, dl.bias)
            ml.forward(0, xd, r, out)
        torch.cuda.synchronize()

    run()  # warm
    m.moe_profile_read()  # drop anything recorded before
    m.moe_profile_enable(True)
    run()
    raw = m.moe_profile_read()
    run()
    stats = m.moe_profile_read_stats()
    m.moe_profile_enable(False)
    assert raw and set(raw) == set(stats), (raw.keys(), stats.keys())
    for k, (total, n) in raw.items():
        t2, med, typ, n2 = stats[k]
        assert n == n2 and n % steps == 0 and n > 0, (k, n, n2)
        assert total > 0 and t2 > 0 and med > 0 and typ > 0, k
        assert typ <= 2 * med * (1 + 1e-9) and med <= t2, (k, med, typ, t2)
    ml.close()


@pytest.mark.parametrize("name,T", [("c2", 1), ("c2", 2), ("c3", 2)])
def test_one_two_token_combine(gpu, name, T):
    """The one/two-token combine sums the terms w*y in fixed point: the combined
    output equals sum_k w[t][k] y(t,k), formed in fp64 from the call's own pair
    outputs, to rounding (no shared expert); a term |w*y| >= 2^21 or not finite
    gives NaN in the affected outputs of that token only and sets MOE_ERR_COMBINE;
    the next call is unaffected and the workspace's leading region is zero again."""
    cfg = synth.CONFIGS[name]
    say(f"[boundary] combine {name} T={T}")
    dl = _layer(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T + 1)
    xh = xh[:T]
    ml = make_layer_api(cfg, dl, T)
    H, K, E = cfg.hidden, cfg.top_k, cfg.n_experts
    ids, w, _, _ = oracle.route(xh, synth.router_f32(cfg), synth.zipf_bias(cfg), K)
    off, sp, _ = oracle.permute(ids, E)
    ref_out, ref_po = _forward(ml, xd, _routing(ml, ids, w, off, sp, gpu), T, H, K, True)
    assert ml.error_word() == 0
    po = ref_po.cpu().numpy().astype(np.float64)
    if cfg.shared_inter == 0:
        for t in range(T):
            want = sum(float(w[t, k]) * po[t * K + k] for k in range(K))
            got = ref_out[t].cpu().numpy().astype(np.float64)
            assert np.linalg.norm(got - want) <= 1e-6 * np.linalg.norm(want), t
    for label, val in (("huge", 1e30), ("nan", float("nan"))):
        w2 = w.copy()
        w2[0, 3] = val
        out, po2 = _forward(ml, xd, _routing(ml, ids, w2, off, sp, gpu), T, H, K, True)
        assert torch.equal(po2, ref_po), label  # the pair outputs do not depend on w
        o0 = out[0].cpu().numpy()
        bad = np.ones(H, bool) if label == "nan" else po[3] != 0
        assert np.isnan(o0[bad]).all() and not np.isnan(o0[~bad]).any(), label
        if T > 1:
            assert torch.equal(out[1:], ref_out[1:]), label
        assert ml.error_word() == moe.MOE_ERR_COMBINE, label
        ml.clear_error()
        out, _ = _forward(ml, xd, _routing(ml, ids, w, off, sp, gpu), T, H, K, True)
        assert torch.equal(out, ref_out), label
        assert ml.error_word() == 0, label
    ctr = ml.ws[:moe.MOE_WS_COUNTER_BYTES].view(torch.int32)
    assert int(torch.count_nonzero(ctr)) == 0
    ml.close()
