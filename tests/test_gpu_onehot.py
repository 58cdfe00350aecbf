"""One-hot codec probes: bit-exact expert outputs from structured weights.

With x = e_j (a single bf16 1.0) the gate and up products are exact: g = q_g[:, j]
* s_g, u = q_u[:, j] * s_u.  The structured experts here use gate codes with
q in {2, 3} and scale 32, so g is 64 or 96 and silu(g) = g / (1 + e^-g) equals g
exactly in fp32 and fp64 (e^-64 is far below half an ulp of 1); up codes are
random over the whole code range with scale 1, so h = g * u is a small integer
(exact in bf16 and fp16); down codes are random with scale 2^-4.  Every sum the
GPU forms is then an integer multiple of 2^-4 well inside fp32's exact range, so
the GPU's pair outputs and combined outputs must equal the oracle's bit for bit,
and both must equal the same values formed from the integer codes the packer was
given.  This pins the GPU unpacker of every code position of the probed columns
(gate and up) and of every code of the down matrices, on each expert path: one
and two tokens, the batched GEMVs (with more positions per expert than one
chunk), and the matrix-core path above 64 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

N_STRUCT = 12  # distinct structured experts; the other table entries repeat them


def _scale_bits(v, f16):
    a = np.array([v], dtype=np.float64)
    return int((synth.f16_bits(a) if f16 else synth.bf16_bits(a))[0])


class StructLayer:
    def __init__(self, cfg, dev, seed):
        rng = np.random.default_rng(seed)
        H, I, bits, G, f16 = cfg.hidden, cfg.inter, cfg.bits, cfg.group, cfg.scale_f16
        z = 1 << (bits - 1)
        self.cfg = cfg
        self.q = []      # (qg, qu, qd) signed integer codes per structured expert
        self.blobs = []  # packed (gate, up, down) per structured expert
        # gate: q in {2, 3} with scale 32 (2-bit codes: q = 1 with scale 64), so g is
        # 64 or 96 and silu(g) = g exactly
        self.sg = 64 if bits == 2 else 32
        s_g, s_u, s_d = (_scale_bits(v, f16) for v in (float(self.sg), 1.0, 2.0 ** -4))
        glo, ghi = (1, 2) if bits == 2 else (2, 4)
        for _ in range(N_STRUCT):
            qg = rng.integers(glo, ghi, size=(I, H), dtype=np.int8)
            qu = rng.integers(-z, z, size=(I, H), dtype=np.int8)
            qd = rng.integers(-z, z, size=(H, I), dtype=np.int8)
            self.q.append((qg, qu, qd))
            self.blobs.append((
                synth.pack_matrix(qg + z, np.full((I, H // G), s_g, np.uint16), bits, G),
                synth.pack_matrix(qu + z, np.full((I, H // G), s_u, np.uint16), bits, G),
                synth.pack_matrix(qd + z, np.full((H, I // G), s_d, np.uint16), bits, G)))
        sizes = [b.nbytes for b in self.blobs[0]]
        self.eb = synth.align(sum(sizes))
        host = np.zeros(N_STRUCT * self.eb, dtype=np.uint8)
        for e, bl in enumerate(self.blobs):
            o = e * self.eb
            for b in bl:
                host[o:o + b.nbytes] = b
                o += b.nbytes
        self.arena = torch.from_numpy(host).to(dev)
        base = self.arena.data_ptr()
        offs = np.cumsum([0] + sizes[:-1])
        self.refs = [tuple(base + (e % N_STRUCT) * self.eb + int(o) for o in offs)
                     for e in range(cfg.n_experts)]

    def exact_y(self, e, js):
        """y of expert e for one-hot tokens at columns js, from the integer codes
        (float64 matrix products of integers below 2^53: exact in any order)"""
        qg, qu, qd = self.q[e % N_STRUCT]
        h = (qg[:, js].astype(np.int64) * self.sg) * qu[:, js]  # [I, n] integers
        return (qd.astype(np.float64) @ h.astype(np.float64)).T / 16.0


def _onehot(T, H, G, odd):
    """columns j_t covering every position inside a group (both codes of each
    pair, the spare-bit pairs of the 3-bit unit) across several groups"""
    ng = H // G
    pos = [((2 * t + 1) if odd else G - 1 - t) % G for t in range(T)]
    js = [G * ((7 * t + 3) % ng) + p for t, p in enumerate(pos)]
    x = np.zeros((T, H), dtype=np.uint16)
    x[np.arange(T), js] = 0x3F80  # bf16 1.0
    return x, np.array(js)


def _routing(T, K, E):
    """expert 0 in every token, expert 1 in every other token, the rest rotating"""
    ids = np.zeros((T, K), dtype=np.int32)
    for t in range(T):
        row = [0] + ([1] if t % 2 == 0 else [])
        c = 2 + (3 * t) % (N_STRUCT - 2)
        while len(row) < K:
            if c not in row:
                row.append(c)
            c = 2 + (c - 1) % (N_STRUCT - 2)
        ids[t] = row
    return ids


_struct = {}


def _struct_layer(name, dev):
    if name not in _struct:
        _struct[name] = StructLayer(synth.CONFIGS[name], dev, seed=100 + len(_struct))
    return _struct[name]


CASES = [("c2", 1, False), ("c2", 2, True), ("c2", 9, False), ("c2", 64, True),
         ("c2", 200, False), ("c1", 1, False), ("c1", 4, True), ("c1", 13, False),
         ("c1", 100, False), ("q2", 1, False), ("q2", 64, True), ("q2", 200, False),
         ("q4", 2, True), ("q4", 9, False), ("q4", 200, False)]


@pytest.mark.parametrize("name,T,odd", CASES)
def test_onehot_probe_bit_exact(gpu, name, T, odd):
    from bit_moe_expert_router_amd import MoELayer, RoutingBuffers
    cfg = synth.CONFIGS[name]
    say(f"[onehot] {name} T={T} bits={cfg.bits} G={cfg.group}")
    H, K, E = cfg.hidden, cfg.top_k, cfg.n_experts
    sl = _struct_layer(name, gpu)
    x, js = _onehot(T, H, cfg.group, odd)
    ids = _routing(T, K, E)
    w = np.full((T, K), 1.0 / K, dtype=np.float32)  # a power of two: combine stays exact
    off, sp, pp = oracle.permute(ids, E)
    ml = MoELayer(H, cfg.inter, E, K, cfg.bits, cfg.group, cfg.scale_f16, 0, T, 1, gpu)
    ml.set_table(0, sl.refs)
    dt = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).to(gpu)
    r = RoutingBuffers(dt(ids, np.int32), dt(w, np.float32), dt(off, np.int32),
                       dt(sp, np.int32), dt(pp, np.int32))
    xd = torch.from_numpy(x.view(np.int16)).to(gpu)
    out = torch.empty((T, H), dtype=torch.float32, device=gpu)
    pair_out = torch.empty((T * K, H), dtype=torch.float32, device=gpu)
    ml.forward(0, xd, r, out, pair_out)
    torch.cuda.synchronize()
    po = pair_out.cpu().numpy().astype(np.float64)
    o = out.cpu().numpy().astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    exact_out = np.zeros((T, H))
    for e in range(N_STRUCT):
        ts, ks = np.nonzero(ids == e)
        if ts.size == 0:
            continue
        y_int = sl.exact_y(e, js[ts])
        g, u, d = sl.blobs[e]
        y_orc = oracle.expert_ffn_multi(xf[ts], g, u, d, H, cfg.inter, cfg.bits, cfg.group,
                                        cfg.scale_f16)
        assert np.array_equal(y_orc, y_int), f"oracle differs from the codes (expert {e})"
        for i, (t, k) in enumerate(zip(ts, ks)):
            assert np.array_equal(po[t * K + k], y_int[i]), (name, T, int(t), int(k), e)
            exact_out[t] += y_int[i] / K
    assert np.array_equal(o, exact_out), (name, T, "combined output")
    say(f"[onehot] {name} T={T}: {T * K} pairs and {T} tokens bit-exact")
    ml.close()
