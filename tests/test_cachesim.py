"""The expert-cache policy replay (host tool) against a plain Python replay of the
same policies on small random traces, plus the bounds every policy obeys (CPU)."""
import numpy as np
import pytest

from bit_moe_expert_router_amd import cachesim


def _random_trace(rng, steps, L, E, kmax):
    return [[rng.choice(E, size=rng.integers(1, kmax + 1), replace=False).tolist()
             for _ in range(L)] for _ in range(steps)]


def _py_replay(steps, L, E, S, policy, decay=0.995):
    """per-step misses of one policy, written from the policy definitions"""
    misses = [0] * len(steps)
    for l in range(L):
        seq = [sorted(set(st[l])) for st in steps]
        resident = []           # slot order matters for CLOCK only
        last, score, ref = {}, {e: 0.0 for e in range(E)}, {}
        hand = 0
        if policy == "static":
            cnt = {e: sum(e in s for s in seq) for e in range(E)}
            resident = sorted(range(E), key=lambda e: (-cnt[e], e))[:S]
        for s, need in enumerate(seq):
            if policy == "lfu":
                for e in score:
                    score[e] *= decay
            for e in need:
                if policy == "lfu":
                    score[e] += 1.0
                if e in resident:
                    if policy == "clock":
                        ref[e] = 1
                    last[e] = s
                    continue
                misses[s] += 1
                last[e] = s
                if policy == "static" or S == 0:
                    continue
                if len(resident) < S:
                    resident.append(e)
                    ref[e] = 1
                    continue
                cands = [v for v in resident if v not in need]
                if not cands:
                    continue
                if policy == "lru":
                    v = min(cands, key=lambda v: (last[v], v))
                elif policy == "lfu":
                    v = min(cands, key=lambda v: (score[v], last[v], v))
                elif policy == "belady":
                    def nxt(v):
                        for t in range(s + 1, len(seq)):
                            if v in seq[t]:
                                return t
                        return float("inf")
                    v = min(cands, key=lambda v: (-nxt(v), v))
                else:  # clock over slot positions
                    v = None
                    for _ in range(2 * S):
                        q = resident[hand]
                        hand = (hand + 1) % S
                        if q in need:
                            continue
                        if ref.get(q, 0):
                            ref[q] = 0
                            continue
                        v = q
                        break
                    if v is None:
                        continue
                i = resident.index(v)
                resident[i] = e
                ref[e] = 1
    return np.array(misses)


@pytest.mark.parametrize("policy", ["static", "lru", "lfu", "belady", "clock"])
@pytest.mark.parametrize("seed,S", [(1, 4), (2, 6), (3, 1), (4, 0)])
def test_replay_matches_python(policy, seed, S):
    rng = np.random.default_rng(seed)
    steps = _random_trace(rng, 150, 2, 12, 4)
    trace, off, L = cachesim.to_csr(steps)
    got = cachesim.simulate(trace, off, L, 12, S, policy, decay=0.9)
    ref = _py_replay(steps, L, 12, S, policy, decay=0.9)
    assert np.array_equal(got, ref), (policy, seed, S)


def test_policy_bounds():
    rng = np.random.default_rng(9)
    # a skewed trace: experts drawn with Zipf-like weights
    E, L = 40, 3
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    steps = [[rng.choice(E, size=6, replace=False, p=p).tolist() for _ in range(L)]
             for _ in range(400)]
    trace, off, L = cachesim.to_csr(steps)
    tot = {pol: int(cachesim.simulate(trace, off, L, E, 12, pol).sum())
           for pol in ("static", "lru", "lfu", "belady", "clock")}
    assert all(tot["belady"] <= v for v in tot.values()), tot  # the optimum
    # with a slot per expert only first uses miss (static pins the most used)
    first = sum(len(set().union(*[set(st[l]) for st in steps])) for l in range(L))
    for pol in ("lru", "lfu", "belady", "clock"):
        assert int(cachesim.simulate(trace, off, L, E, E, pol).sum()) == first, pol
    assert int(cachesim.simulate(trace, off, L, E, E, "static").sum()) == 0
    # no slots: every pick misses
    assert int(cachesim.simulate(trace, off, L, E, 0, "lru").sum()) == len(trace)
    # LRU and Belady are stack policies: more slots never miss more
    for pol in ("lru", "belady"):
        m = [int(cachesim.simulate(trace, off, L, E, S, pol).sum()) for S in (6, 8, 12, 20)]
        assert m == sorted(m, reverse=True), (pol, m)
