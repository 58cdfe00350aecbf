"""Seeded input generator: published SplitMix64 vector, determinism, stream
independence and value ranges (CPU)."""
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed1234567.txt")


def test_splitmix64_published_vector():
    want = [int(l) for l in open(GOLD) if l.strip() and not l.startswith("#")]
    # draw(key, i) is output i of a SplitMix64 generator whose state starts at key
    got = [synth.draw(1234567, i) for i in range(len(want))]
    assert got == want


def test_codes_deterministic_and_streams_distinct():
    a = synth.codes_bytes(4096, 2, 0, 5, 1)
    b = synth.codes_bytes(4096, 2, 0, 5, 1)
    assert np.array_equal(a, b)
    for other in [(3, 0, 5, 1), (2, 1, 5, 1), (2, 0, 6, 1), (2, 0, 5, 2)]:
        assert not np.array_equal(a, synth.codes_bytes(4096, *other))
    # prefix property: a longer fill starts with the shorter one
    assert np.array_equal(synth.codes_bytes(8192, 2, 0, 5, 1)[:4096], a)


def test_code_bytes_uniform():
    a = synth.codes_bytes(1 << 20, 9, 0, 0, 0)
    bits = np.unpackbits(a)
    assert abs(bits.mean() - 0.5) < 2e-3
    counts = np.bincount(a, minlength=256)
    assert counts.min() > 0.8 * counts.mean()


def test_scales_range_and_rounding():
    for f16 in (False, True):
        s = synth.scales_u16(100000, 2, 0, 3, 0, f16)
        v = (s.view(np.float16).astype(np.float64) if f16 else synth.bf16_to_f32(s).astype(np.float64))
        assert v.min() >= 0.01 * (1 - 2 ** -8) and v.max() <= 0.05 * (1 + 2 ** -8)
        assert abs(v.mean() - 0.03) < 5e-4


def test_normals_moments():
    x = synth.bf16_to_f32(synth.normal_bf16(200000, 1, 0, synth.SYN_X, 1.0)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    r = synth.normal_f32(200000, 1, 0, synth.SYN_ROUTER, 0.02).astype(np.float64)
    assert abs(r.std() - 0.02) < 3e-4


def test_permutation_and_zipf_bias():
    p = synth.permutation(288, 2, 0, synth.SYN_BIAS_PERM)
    assert sorted(p.tolist()) == list(range(288))
    cfg = synth.CONFIGS["c2"]
    b = synth.zipf_bias(cfg)
    # exp(bias) is proportional to rank^-1.1 for ranks 1..288
    ranks = np.sort(np.exp(-b.astype(np.float64) / 1.1))
    assert np.allclose(ranks, np.arange(1, 289), rtol=1e-5)
    assert synth.zipf_bias(synth.CONFIGS["c1"]) is None


def test_shared_weights_moments():
    cfg = synth.CONFIGS["c3"].with_(hidden=512, shared_inter=256)
    g, u, d = synth.shared_weights(cfg)
    v = synth.bf16_to_f32(g).astype(np.float64)
    assert abs(v.std() - 0.0754) < 2e-3
    assert not np.array_equal(g, u)
