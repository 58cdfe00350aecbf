"""Oracle routing pinned by brute force, forced ties, closed forms and a library
softmax, and grouping pinned by brute force (CPU)."""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


def _inputs(cfg, tokens=None):
    return (synth.x_bf16(cfg, tokens), synth.router_f32(cfg), synth.zipf_bias(cfg))


def test_topk_brute_force_c1():
    """the chosen set maximises the sum of logits over all C(16,2) subsets and is
    listed by descending logit"""
    cfg = synth.CONFIGS["c1"]
    x, Wr, b = _inputs(cfg, tokens=64)
    ids, w, gap, logits = oracle.route(x, Wr, b, cfg.top_k)
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(cfg.n_experts), cfg.top_k),
                   key=lambda s: (sum(logits[t, list(s)]), [-e for e in s]))
        assert sorted(ids[t].tolist()) == sorted(best)
        assert logits[t, ids[t, 0]] >= logits[t, ids[t, 1]]


def test_logits_match_definition():
    cfg = synth.CONFIGS["c2"]
    x, Wr, b = _inputs(cfg, tokens=2)
    _, _, _, logits = oracle.route(x, Wr, b, cfg.top_k)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = xf @ Wr.astype(np.float64).T + b.astype(np.float64)
    assert np.allclose(logits, ref, rtol=0, atol=1e-12)


def test_logits_one_hot_closed_form():
    """x = c * e_j (one nonzero bf16 entry) makes every product but one zero, so
    l[e] = c * Wr[e, j] + bias[e] exactly: the fp64 product of a bf16 and an fp32
    value is exact, and so is the sum of two such values of nearby magnitude.  A
    dropped bias, a transposed router or a wrong column fails here."""
    cfg = synth.CONFIGS["c2"]
    Wr, b = synth.router_f32(cfg), synth.zipf_bias(cfg)
    H = cfg.hidden
    cols = [0, 1, 127, 128, 2559, H - 1]
    vals = [1.0, -2.5, 0.375, -1.0, 3.0, 0.0078125]
    x = np.zeros((len(cols), H), dtype=np.uint16)
    for t, (j, c) in enumerate(zip(cols, vals)):
        x[t, j] = synth.bf16_bits(np.array([c]))[0]
    _, _, _, logits = oracle.route(x, Wr, b, cfg.top_k)
    for t, (j, c) in enumerate(zip(cols, vals)):
        expect = c * Wr[:, j].astype(np.float64) + b.astype(np.float64)
        assert np.array_equal(logits[t], expect), (t, j)


def test_logits_dyadic_exact_sum():
    """x entries in {0, +-1/2, +-1, +-2} and router entries k/1024 with small
    integers k: every partial sum is a multiple of 2^-11 far below 2^53, so the
    fp64 logits are the exact rational sums, computed here with Python integers
    (order-free).  Pins the whole reduction (every column, every row)."""
    rng = np.random.default_rng(7)
    T, H, E = 5, 512, 24
    xv = rng.choice(np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0]), size=(T, H))
    x = synth.bf16_bits(xv)
    kr = rng.integers(-300, 301, size=(E, H))
    Wr = (kr / 1024.0).astype(np.float32)
    kb = rng.integers(-5000, 5001, size=E)
    bias = (kb / 1024.0).astype(np.float32)
    _, _, _, logits = oracle.route(x, Wr, bias, 4)
    xi = (xv * 2).astype(np.int64)  # x * 2, integers
    for t in range(T):
        for e in range(E):
            num = sum(int(xi[t, h]) * int(kr[e, h]) for h in range(H)) + 2 * int(kb[e])
            assert logits[t, e] == num / 2048.0, (t, e)


def test_tie_break_lower_id_first():
    """duplicated router rows give exactly equal logits; the lower id wins and is
    listed first"""
    cfg = synth.CONFIGS["c1"]
    x, Wr, _ = _inputs(cfg, tokens=8)
    Wr = Wr.copy()
    xf = synth.bf16_to_f32(x).astype(np.float64)
    for t in range(8):
        top = int(np.argmax(xf[t] @ Wr.astype(np.float64).T))
        W2 = Wr.copy()
        W2[[3, 11]] = Wr[top]  # experts 3 and 11 tie with the best one
        W2[top] = Wr[top]
        ids, _, _, logits = oracle.route(x[t:t + 1], W2, None, 2)
        tied = sorted({3, 11, top})
        assert ids[0].tolist() == tied[:2]
        assert logits[0, 3] == logits[0, 11]


def test_weights_closed_form_k2():
    """K = 2: w0 = logistic(l0 - l1), w1 = 1 - w0"""
    cfg = synth.CONFIGS["c1"]
    x, Wr, b = _inputs(cfg, tokens=32)
    ids, w, _, logits = oracle.route(x, Wr, b, 2)
    for t in range(32):
        d = logits[t, ids[t, 0]] - logits[t, ids[t, 1]]
        assert math.isclose(w[t, 0], 1.0 / (1.0 + math.exp(-d)), rel_tol=1e-14)
        assert math.isclose(w[t, 1], 1.0 / (1.0 + math.exp(d)), rel_tol=1e-14)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_weights_equal_restricted_softmax(name):
    cfg = synth.CONFIGS[name]
    x, Wr, b = _inputs(cfg)
    ids, w, _, logits = oracle.route(x, Wr, b, cfg.top_k)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)  # softmax over all experts
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending logits -> descending weights


@pytest.mark.parametrize("name,zipf,tokens", [("c1", False, None), ("c2", True, None),
                                              ("c3", True, None), ("c5", True, None),
                                              ("c5", False, None), ("q2", True, 65),
                                              ("q4", True, 65), ("c3", True, 300),
                                              ("c1", False, 300), ("c2", True, 65)])
def test_config_seeds_have_no_near_ties(name, zipf, tokens):
    """Routing ids are compared bit-exactly against the GPU, so every token of the
    fixed seeds must keep its K-th pick clear of the (K+1)-th, and the picks clear
    of each other (their order is the output order), by far more than any fp64
    summation-order difference (< 1e-12 here)."""
    cfg = synth.CONFIGS[name].with_(zipf=zipf)
    x, Wr, b = _inputs(cfg, tokens)
    ids, _, gap, logits = oracle.route(x, Wr, b, cfg.top_k)
    assert gap.min() > 1e-9, (name, gap.min())
    top = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    assert np.all(-np.diff(top, axis=1) > 1e-9), name


def test_zipf_skews_routing():
    cfg = synth.CONFIGS["c3"]
    x, Wr, b = _inputs(cfg, tokens=256)
    ids, _, _, _ = oracle.route(x, Wr, b, cfg.top_k)
    ids_u, _, _, _ = oracle.route(x, Wr, None, cfg.top_k)
    # skewed routing concentrates picks on fewer distinct experts
    assert len(np.unique(ids)) < len(np.unique(ids_u))


# ------------------------------------------------------------------ grouping
def _brute_group(ids, E):
    flat = ids.reshape(-1)
    sp = [p for e in range(E) for p in range(flat.size) if flat[p] == e]
    counts = [int((flat == e).sum()) for e in range(E)]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), np.array(sp, np.int32)


@pytest.mark.parametrize("T,K,E", [(1, 8, 288), (8, 8, 288), (4, 2, 16), (37, 3, 5)])
def test_permute_brute_force(T, K, E):
    rng = np.random.default_rng(T * 100 + K)
    ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    off, sp, pp = oracle.permute(ids, E)
    off_b, sp_b = _brute_group(ids, E)
    assert np.array_equal(off, off_b) and np.array_equal(sp, sp_b)
    assert np.array_equal(pp[sp], np.arange(T * K))       # pair_pos o sorted_pairs = id
    assert np.array_equal(sp[pp], np.arange(T * K))
    for e in range(E):                                     # stable within an expert
        seg = sp[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(ids.reshape(-1)[seg] == e)


def test_permute_skips_invalid_ids():
    ids = np.array([[0, 5], [7, -1], [3, 0]], dtype=np.int32)
    off, sp, pp = oracle.permute(ids, 6)
    assert off[-1] == 4
    assert pp[2] == -1 and pp[3] == -1
    assert sp.tolist() == [0, 5, 4, 1]
