"""Exact ties in the router logits on every routing path of the HIP library.

Duplicated router rows (and bias entries) give two experts exactly equal logits
on both sides: each side computes the two sums in the same order.  The reading
taken for such ties is that the lower logical expert id wins and is listed
first (the pages print no router; the tie rule is part of the plainest
deterministic top-k).  The cases reach each routing path the library has: one
launch for one or two tokens, the small-batch logits + top-k/grouping pair (up
to 16 tokens), the small-batch logits with the one-wave-per-token top-k and the
single-wave grouping (17..32 tokens), the fp64 matrix-core logits (above 32
tokens) and the multi-block grouping (more than 4,096 pairs).  Ids, offsets,
sorted pairs and pair positions must match the oracle bit for bit, weights to
fp32 rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import make_layer_api, say
from synth.device import DeviceLayer, x_device

pytestmark = pytest.mark.gpu

W_TOL = 2e-7
NEAR = 1e-9  # logits closer than this but not equal would make the comparison ill-posed

_layers = {}


def _layer(name, dev):
    if name not in _layers:
        _layers[name] = DeviceLayer.generate(synth.CONFIGS[name], 0, dev)
    return _layers[name]


def tied_router(cfg, xh, n_src):
    """router and bias with the rows of the n_src most picked experts copied to
    other ids (half of them lower, half higher), and each token's K-th pick copied
    to an id on the other side of it; returns (Wr, bias, pairs copied)"""
    Wr = synth.router_f32(cfg).copy()
    b = synth.zipf_bias(cfg)
    b = None if b is None else b.copy()
    ids, _, _, _ = oracle.route(xh, Wr, b, cfg.top_k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.n_experts)
    srcs = [int(e) for e in np.argsort(-counts, kind="stable")[:n_src]]
    srcs += [int(ids[t, -1]) for t in range(min(2, ids.shape[0])) if int(ids[t, -1]) not in srcs]
    used = set(srcs)
    copies = []
    for i, s in enumerate(srcs):
        want_lower = i % 2 == 0
        cand = range(s - 1, -1, -1) if want_lower else range(s + 1, cfg.n_experts)
        d = next((c for c in cand if c not in used), None)
        if d is None:
            cand = range(s + 1, cfg.n_experts) if want_lower else range(s - 1, -1, -1)
            d = next(c for c in cand if c not in used)
        used.add(d)
        Wr[d] = Wr[s]
        if b is not None:
            b[d] = b[s]
        copies.append((s, d))
    return Wr, b, copies


CASES = [("c1", 1), ("c2", 1), ("c2", 2), ("c2", 3), ("c2", 4), ("c2", 5), ("c3", 16), ("c3", 24), ("c3", 37),
         ("c3", 300), ("c5", 8192)]


def _check_route(gpu, cfg, dl, xd, T, Wr, b, ids, w):
    ml = make_layer_api(cfg, dl, T)
    wr_d = torch.from_numpy(Wr).to(gpu)
    b_d = None if b is None else torch.from_numpy(b).to(gpu)
    r = ml.route(xd, wr_d, b_d)
    torch.cuda.synchronize()
    assert np.array_equal(r.topk_ids.cpu().numpy(), ids), "ids differ"
    wg = r.topk_w.cpu().numpy()
    assert np.all(np.abs(wg - w) <= W_TOL * np.maximum(w, 1e-30) + 1e-12)
    off, sp, pp = oracle.permute(ids, cfg.n_experts)
    assert np.array_equal(r.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(r.sorted_pairs.cpu().numpy()[:off[-1]], sp)
    assert np.array_equal(r.pair_pos.cpu().numpy(), pp)
    ml.close()


@pytest.mark.parametrize("name,T", CASES)
def test_routing_exact_ties(gpu, name, T):
    say(f"[ties] {name} T={T}")
    cfg = synth.CONFIGS[name]
    dl = _layer(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    Wr, b, copies = tied_router(cfg, xh, 4 if cfg.n_experts > 16 else 2)
    ids, w, gap, logits = oracle.route(xh, Wr, b, cfg.top_k)
    # the comparison is well posed: among each token's K+1 largest logits two
    # values are either exactly equal or clearly apart
    srt = -np.sort(-logits, axis=1)[:, :cfg.top_k + 1]
    d = -np.diff(srt, axis=1)
    assert np.all((d == 0) | (d > NEAR)), name
    n_tied = int(np.sum(np.any(d == 0, axis=1)))
    assert n_tied > 0, "no token has a tie among its leading logits"
    _check_route(gpu, cfg, dl, xd, T, Wr, b, ids, w)
    # the lower id of each copied pair wins wherever the two tie for a place
    for s, dd in copies:
        lo, hi = min(s, dd), max(s, dd)
        has_hi = np.any(ids == hi, axis=1)
        assert np.all(np.any(ids[has_hi] == lo, axis=1)), (s, dd)
    say(f"[ties] {name} T={T}: {n_tied} tokens with a tie among their leading logits")


MASS = [("c1", 1, "all"), ("c2", 1, "all"), ("c2", 1, "blocks"), ("c2", 2, "blocks"),
        ("c2", 2, "all"), ("c2", 4, "blocks"), ("c2", 3, "all"), ("c3", 5, "blocks"), ("c3", 9, "all"), ("c3", 37, "blocks"),
        ("c3", 300, "all")]


@pytest.mark.parametrize("name,T,mode", MASS)
def test_routing_mass_ties(gpu, name, T, mode):
    """Many experts with equal logits: every router row (and bias entry) the same
    ("all": each token's logits are all equal, the picks are ids 0..K-1 with
    weights 1/K), or the same within blocks of consecutive ids ("blocks": the
    leading block's ids tie, the lowest of them are picked in id order).  These
    reach the top-k's one-round-at-a-time path (more equal leading keys than a
    wave holds) and its ranking of equal candidates."""
    say(f"[mass ties] {name} T={T} {mode}")
    cfg = synth.CONFIGS[name]
    dl = _layer(name, gpu)
    xh, xd = x_device(cfg, gpu, tokens=T)
    Wr = synth.router_f32(cfg).copy()
    b = synth.zipf_bias(cfg)
    b = None if b is None else b.copy()
    blk = cfg.n_experts if mode == "all" else max(cfg.n_experts // 12, cfg.top_k + 1)
    src = (np.arange(cfg.n_experts) // blk) * blk
    Wr = np.ascontiguousarray(Wr[src])
    if b is not None:
        b = np.ascontiguousarray(b[src])
    ids, w, gap, logits = oracle.route(xh, Wr, b, cfg.top_k)
    if mode == "all":
        assert np.array_equal(ids, np.tile(np.arange(cfg.top_k), (T, 1)))
        assert np.allclose(w, 1.0 / cfg.top_k, rtol=1e-15)
    _check_route(gpu, cfg, dl, xd, T, Wr, b, ids, w)
