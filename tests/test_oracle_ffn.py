"""Oracle experts, combine and stack glue pinned by an independent dense-gating
formulation, closed forms and one-hot probes, plus the layer invariants (CPU)."""
import math

import numpy as np
import pytest

import oracle
import synth


def _silu(z):
    return z / (1.0 + np.exp(-z))


class DenseLayer:
    """A small MoE layer held twice: as unsigned codes and scales (for the dense
    numpy formulation) and as packed blobs (for the oracle)."""

    def __init__(self, H, I, E, bits, G, f16, seed, shared_inter=0):
        rng = np.random.default_rng(seed)
        self.H, self.I, self.E, self.bits, self.G, self.f16 = H, I, E, bits, G, f16
        self.W = []      # dequantised (gate, up, down) per expert, from codes and scales
        self.blobs = []  # packed (gate, up, down) per expert
        for e in range(E):
            mats, blobs = [], []
            for rows, cols in ((I, H), (I, H), (H, I)):
                c = rng.integers(0, 1 << bits, size=(rows, cols))
                s = rng.uniform(0.01, 0.05, size=(rows, cols // G))
                sb = synth.f16_bits(s) if f16 else synth.bf16_bits(s)
                sv = (sb.view(np.float16) if f16 else synth.bf16_to_f32(sb)).astype(np.float64)
                mats.append((c - (1 << (bits - 1))) * np.repeat(sv, G, axis=1))
                blobs.append(synth.pack_matrix(c, sb, bits, G))
            self.W.append(mats)
            self.blobs.append(blobs)
        self.shared = None
        if shared_inter:
            sw = [synth.bf16_bits(rng.uniform(-0.13, 0.13, size=sh))
                  for sh in ((shared_inter, H), (shared_inter, H), (H, shared_inter))]
            self.shared = tuple(sw)

    def tables(self):
        return ([b[0] for b in self.blobs], [b[1] for b in self.blobs], [b[2] for b in self.blobs])

    def dense_out(self, xf, logits, K):
        """out[t] = sum_e G[t,e] * FFN_e(x_t) over ALL experts, G the softmax over
        all experts masked to the top-K set and renormalised; shared expert added"""
        T = xf.shape[0]
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        Gm = np.zeros_like(p)
        for t in range(T):
            top = np.argsort(-logits[t], kind="stable")[:K]
            Gm[t, top] = p[t, top] / p[t, top].sum()
        out = np.zeros((T, self.H))
        for e in range(self.E):
            g, u, d = self.W[e]
            y = (_silu(xf @ g.T) * (xf @ u.T)) @ d.T
            out += Gm[:, [e]] * y
        if self.shared is not None:
            sg, su, sd = (synth.bf16_to_f32(a).astype(np.float64) for a in self.shared)
            out += (_silu(xf @ sg.T) * (xf @ su.T)) @ sd.T
        return out


@pytest.mark.parametrize("bits,G,f16,shared", [(4, 32, True, 0), (3, 128, False, 0),
                                               (3, 128, False, 128), (2, 128, False, 0),
                                               (4, 128, False, 0)])
def test_layer_equals_dense_gating(bits, G, f16, shared):
    H, I, E, K, T = 256, 128, 16, 2, 6
    L = DenseLayer(H, I, E, bits, G, f16, seed=11 + bits, shared_inter=shared)
    cfg = synth.CONFIGS["c1"]
    x = synth.x_bf16(cfg, tokens=T)
    Wr = synth.router_f32(cfg)
    ids, w, _, logits = oracle.route(x, Wr, None, K)
    out, pair_out = oracle.moe_layer(x, ids, w, *L.tables(), I, bits, G, f16, L.shared)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = L.dense_out(xf, logits, K)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)
    # pair outputs are the unweighted expert outputs
    for t in range(T):
        for k in range(K):
            g, u, d = L.W[ids[t, k]]
            y = (_silu(g @ xf[t]) * (u @ xf[t])) @ d.T
            assert np.allclose(pair_out[t * K + k], y, rtol=1e-12, atol=1e-12)


def test_one_hot_probe_reads_columns():
    """x = e_j gives gate.x = column j of the dequantised gate matrix, exactly"""
    L = DenseLayer(256, 128, 1, 3, 128, False, seed=5)
    for j in (0, 1, 127, 128, 200, 255):
        v = np.zeros(256)
        v[j] = 1.0
        y = oracle.matvec(L.blobs[0][0], 128, 256, 3, 128, False, v)
        assert np.array_equal(y, L.W[0][0][:, j])


def test_zero_point_codes_give_zero_output():
    """up codes at the zero point (q = 0) make h = 0, so y = 0 exactly; gate codes
    at the zero point give silu(0) = 0 and y = 0"""
    H, I, bits, G = 256, 128, 3, 128
    rng = np.random.default_rng(3)
    zero = np.full((I, H), 4)
    s = synth.bf16_bits(rng.uniform(0.01, 0.05, size=(I, H // G)))
    sd = synth.bf16_bits(rng.uniform(0.01, 0.05, size=(H, I // G)))
    rnd = lambda r, c: rng.integers(0, 8, size=(r, c))
    x = synth.bf16_to_f32(synth.x_bf16(synth.CONFIGS["c1"], 1)[0]).astype(np.float64)
    for gate_c, up_c in ((rnd(I, H), zero), (zero, rnd(I, H))):
        y = oracle.expert_ffn(x, synth.pack_matrix(gate_c, s, bits, G),
                              synth.pack_matrix(up_c, s, bits, G),
                              synth.pack_matrix(rnd(H, I), sd, bits, G), H, I, bits, G, False)
        assert np.all(y == 0.0)


def test_constant_codes_closed_form():
    """all codes c and one scale s: gate.x = (c-4)*s*sum(x); checks the whole
    SwiGLU chain against its closed form"""
    H, I, bits, G = 256, 128, 3, 128
    s = synth.bf16_bits(np.array([0.03125]))[0]  # exact in bf16
    sv = 0.03125
    mk = lambda c, r, k: synth.pack_matrix(np.full((r, k), c), np.full((r, k // G), s), bits, G)
    x = synth.bf16_to_f32(synth.x_bf16(synth.CONFIGS["c1"], 1)[0]).astype(np.float64)
    y = oracle.expert_ffn(x, mk(7, I, H), mk(5, I, H), mk(2, H, I), H, I, bits, G, False)
    g = 3 * sv * x.sum()
    u = 1 * sv * x.sum()
    h = g / (1 + math.exp(-g)) * u
    want = -2 * sv * I * h
    assert np.allclose(y, want, rtol=1e-12)


# ------------------------------------------------------------------ invariants
def _c1_layer():
    cfg = synth.CONFIGS["c1"]
    blobs = [synth.expert_blob(cfg, 0, e) for e in range(cfg.n_experts)]
    off = synth.matrix_offsets(cfg)
    tabs = ([b[off[0]:off[1]] for b in blobs], [b[off[1]:off[2]] for b in blobs],
            [b[off[2]:] for b in blobs])
    return cfg, tabs


def test_invariant_token_reorder():
    cfg, tabs = _c1_layer()
    x = synth.x_bf16(cfg, tokens=5)
    ids, w, _, _ = oracle.route(x, synth.router_f32(cfg), None, cfg.top_k)
    out, _ = oracle.moe_layer(x, ids, w, *tabs, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16)
    perm = np.array([3, 0, 4, 1, 2])
    ids2, w2, _, _ = oracle.route(x[perm], synth.router_f32(cfg), None, cfg.top_k)
    out2, _ = oracle.moe_layer(x[perm], ids2, w2, *tabs, cfg.inter, cfg.bits, cfg.group,
                               cfg.scale_f16)
    assert np.array_equal(ids2, ids[perm]) and np.array_equal(out2, out[perm])


def test_invariant_zero_weight_pair():
    cfg, tabs = _c1_layer()
    x = synth.x_bf16(cfg, tokens=3)
    ids, w, _, _ = oracle.route(x, synth.router_f32(cfg), None, cfg.top_k)
    w0 = w.copy()
    w0[1, 1] = 0.0
    out0, _ = oracle.moe_layer(x, ids, w0, *tabs, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16)
    ids_d = ids.copy()
    ids_d[1, 1] = -1  # the pair dropped
    outd, _ = oracle.moe_layer(x, ids_d, w0, *tabs, cfg.inter, cfg.bits, cfg.group,
                               cfg.scale_f16)
    assert np.array_equal(out0, outd)


def test_invariant_remap():
    """logical id -> any physical placement: results depend on the logical id only"""
    cfg, tabs = _c1_layer()
    x = synth.x_bf16(cfg, tokens=4)
    ids, w, _, _ = oracle.route(x, synth.router_f32(cfg), None, cfg.top_k)
    out, _ = oracle.moe_layer(x, ids, w, *tabs, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16)
    perm = synth.permutation(cfg.n_experts, 9, 0, synth.SYN_SLOT_PERM)
    arena = [[None] * cfg.n_experts for _ in range(3)]
    for e in range(cfg.n_experts):  # copy each expert into slot perm[e]
        for m in range(3):
            arena[m][perm[e]] = tabs[m][e].copy()
    remapped = tuple([arena[m][perm[e]] for e in range(cfg.n_experts)] for m in range(3))
    out2, _ = oracle.moe_layer(x, ids, w, *remapped, cfg.inter, cfg.bits, cfg.group,
                               cfg.scale_f16)
    assert np.array_equal(out, out2)


# ------------------------------------------------------------------ stack glue
@pytest.mark.parametrize("c", [1.0, -3.5, 1e-4, 250.0])
def test_rmsnorm_constant_vector(c):
    H = 512
    r = oracle.rmsnorm(np.full(H, c), 1e-6)
    want = math.copysign(1.0, c) / math.sqrt(1.0 + 1e-6 / (c * c))
    assert np.allclose(r, want, rtol=1e-15)


def test_rmsnorm_unit_rms():
    x = np.random.default_rng(0).normal(size=5120) * 7
    r = oracle.rmsnorm(x, 0.0)
    assert math.isclose(np.sqrt(np.mean(r * r)), 1.0, rel_tol=1e-14)


def test_double_to_bf16_rne():
    cases = {1.0: 0x3F80, -2.0: 0xC000, 1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82,
             1 + 2 ** -8 + 2 ** -30: 0x3F81, 0.0: 0, 3.0: 0x4040}
    for v, bits in cases.items():
        assert oracle.double_to_bf16(v) == bits, (v, hex(oracle.double_to_bf16(v)))
    assert oracle.bf16_to_double(0x3F81) == 1 + 2 ** -7
    assert oracle.f16_to_double(0x3C00) == 1.0 and oracle.f16_to_double(0x0001) == 2 ** -24


def test_expert_ffn_multi_equals_single():
    """the batched form applies the same per-vector arithmetic: bit-identical rows"""
    H, I = 256, 128
    L = DenseLayer(H, I, 2, 3, 128, False, seed=5)
    cfg = synth.CONFIGS["c1"]
    x = synth.bf16_to_f32(synth.x_bf16(cfg, tokens=5)).astype(np.float64)
    g, u, d = L.blobs[1]
    Y = oracle.expert_ffn_multi(x, g, u, d, H, I, 3, 128, False)
    for j in range(5):
        assert np.array_equal(Y[j], oracle.expert_ffn(x[j], g, u, d, H, I, 3, 128, False))
