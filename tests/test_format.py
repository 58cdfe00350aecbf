"""Packed weight format as read by the oracle: every stored bit belongs to exactly
one code bit, paired codes share bit offsets in the two 16-bit halves, tiles and
chunks map to rows and groups, the packer round-trips, and the byte sizes match
the ~9 MB-per-expert figure (CPU)."""
import numpy as np
import pytest

import oracle
import synth


def _single_unit_matrix(bits, G, word, bit):
    """64 x G matrix (one tile): only `bit` of `word` of lane 0's unit is set."""
    lay = synth.matrix_layout(64, G, bits, G)
    blob = np.zeros(lay.nbytes, dtype=np.uint8)
    j, wi = divmod(word, 4)
    off = j * 1024 + 0 * 16 + 4 * wi
    v = np.frombuffer(blob[off:off + 4].tobytes(), dtype=np.uint32).copy()
    v[0] |= np.uint32(1 << bit)
    blob[off:off + 4] = v.view(np.uint8)
    return blob


CODECS = [(3, 128), (4, 32), (2, 128), (4, 128)]


@pytest.mark.parametrize("bits,G", CODECS)
def test_bit_bijection(bits, G):
    nwords = bits * G // 32
    seen = {}
    for word in range(nwords):
        for bit in range(32):
            blob = _single_unit_matrix(bits, G, word, bit)
            codes = [oracle.code(blob, 64, G, bits, G, 0, 0, i) for i in range(G)]
            nz = [(i, c) for i, c in enumerate(codes) if c]
            assert len(nz) == 1, (word, bit, nz)
            i, c = nz[0]
            assert c & (c - 1) == 0  # exactly one code bit
            key = (i, c.bit_length() - 1)
            assert key not in seen
            seen[key] = (word, bit)
            # no other lane's code moves
            assert oracle.code(blob, 64, G, bits, G, 1, 0, i) == 0
    assert len(seen) == G * bits


@pytest.mark.parametrize("bits,G", CODECS)
def test_pairs_share_offsets_in_halves(bits, G):
    """codes 2P and 2P+1 sit at the same bit offsets of the low and high halves
    of the same word(s)"""
    where = {}
    nwords = bits * G // 32
    for word in range(nwords):
        for bit in range(32):
            blob = _single_unit_matrix(bits, G, word, bit)
            for i in range(G):
                c = oracle.code(blob, 64, G, bits, G, 0, 0, i)
                if c:
                    where[(i, c.bit_length() - 1)] = (word, bit)
    for P in range(G // 2):
        for b in range(bits):
            w0, b0 = where[(2 * P, b)]
            w1, b1 = where[(2 * P + 1, b)]
            assert w0 == w1 and b0 < 16 and b1 == b0 + 16


@pytest.mark.parametrize("bits,G,N,Kd", [(3, 128, 128, 512), (4, 32, 192, 96),
                                         (2, 128, 128, 384), (4, 128, 64, 256)])
def test_packer_roundtrip_and_tiles(bits, G, N, Kd):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 1 << bits, size=(N, Kd))
    scales = synth.bf16_bits(rng.uniform(0.01, 0.05, size=(N, Kd // G)))
    blob = synth.pack_matrix(codes, scales, bits, G)
    assert blob.size == oracle.matrix_bytes(N, Kd, bits, G)
    for n in range(0, N, 7):
        for g in range(Kd // G):
            got = [oracle.code(blob, N, Kd, bits, G, n, g, i) for i in range(G)]
            assert got == codes[n, g * G:(g + 1) * G].tolist()
            assert oracle.scale(blob, N, Kd, bits, G, False, n, g) == float(
                synth.bf16_to_f32(scales[n, g]))
    W = oracle.dequant(blob, N, Kd, bits, G, False)
    ref = (codes - (1 << (bits - 1))) * np.repeat(
        synth.bf16_to_f32(scales).astype(np.float64), G, axis=1)
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("bits,G,N,Kd", [(3, 128, 192, 384), (4, 32, 128, 96)])
def test_scale_tile_order(bits, G, N, Kd):
    """the scale stored at scales_off + 2*(t*64 + u) (tile t = (n/64)*ng + g,
    u = n % 64) is the scale of row n and group g, and of no other (row, group)"""
    lay = synth.matrix_layout(N, Kd, bits, G)
    ng = Kd // G
    one = 0x3F80  # bf16 1.0
    for n, g in [(0, 0), (1, 0), (63, ng - 1), (64, 0), (N - 1, ng - 1), (70, ng // 2)]:
        blob = np.zeros(lay.nbytes, dtype=np.uint8)
        t, u = (n // 64) * ng + g, n % 64
        off = lay.scales_off + 2 * (t * 64 + u)
        blob[off:off + 2] = np.array([one], dtype=np.uint16).view(np.uint8)
        for nn in range(N):
            for gg in range(ng):
                want = 1.0 if (nn, gg) == (n, g) else 0.0
                assert oracle.scale(blob, N, Kd, bits, G, False, nn, gg) == want, (n, g, nn, gg)


def test_tile_chunk_addressing():
    """a bit set in chunk j of tile t at lane u lands in row 64*(t // ng) + u,
    group t % ng"""
    bits, G, N, Kd = 3, 128, 128, 256
    lay = synth.matrix_layout(N, Kd, bits, G)
    ng = Kd // G
    for t in range(4):
        for j in range(3):
            for u in (0, 5, 63):
                blob = np.zeros(lay.nbytes, dtype=np.uint8)
                blob[(t * 3 + j) * 1024 + 16 * u] = 2  # bit 1 of word 4j: field 0 of pair 5*4j
                n, g = 64 * (t // ng) + u, t % ng
                W = oracle.dequant_row(blob, N, Kd, bits, G, False, n)
                codes = [oracle.code(blob, N, Kd, bits, G, n, g, i) for i in range(G)]
                assert codes.count(1) == 1 and codes.index(1) == 2 * (5 * 4 * j)
                # every other row reads all-zero codes
                other = (n + 1) % N
                assert all(oracle.code(blob, N, Kd, bits, G, other, gg, i) == 0
                           for gg in range(ng) for i in range(0, G, 9))
                del W


def test_expert_sizes():
    assert synth.expert_bytes(synth.CONFIGS["c2"]) == 9_216_000
    assert synth.expert_bytes(synth.CONFIGS["c1"]) == 55_296
    g, u, d = synth.expert_layouts(synth.CONFIGS["c2"])
    assert g.codes_bytes == 2_949_120 and g.scales_bytes == 122_880 and g.nbytes == 3_072_000
    # ~9 MiB per expert at ~3 bpw on the pages: ours is 3.125 bits per weight
    nw = 3 * 5120 * 1536
    assert abs(synth.expert_bytes(synth.CONFIGS["c2"]) * 8 / nw - 3.125) < 1e-12


def test_generated_blob_matches_generator_streams():
    cfg = synth.CONFIGS["c1"]
    blob = synth.expert_blob(cfg, 0, 3)
    g, u, d = synth.expert_layouts(cfg)
    off = synth.matrix_offsets(cfg)
    assert np.array_equal(blob[off[1]:off[1] + u.codes_bytes],
                          synth.codes_bytes(u.codes_bytes, cfg.seed, 0, 3, 1))
    sc = blob[off[2] + d.scales_off: off[2] + d.scales_off + d.scales_bytes].view(np.uint16)
    assert np.array_equal(sc, synth.scales_u16(d.rows * d.n_groups, cfg.seed, 0, 3, 2, True))
