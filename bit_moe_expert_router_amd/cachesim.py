"""Expert-cache policy replay (host tool over ``libcachesim.so``, built from
``host/cachesim.c``): misses per step of the static, LRU, LFU (decay per step),
Belady and CLOCK policies with S slots per layer, over a routing trace.  The
pages compare these policies by misses per token on recorded traces (page
"GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO 6000 - GPU expert cache, host-RAM
streaming", field config.expert_cache.policy_data); the policy semantics are in
the C source.  Marshalling only."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

STATIC, LRU, LFU, BELADY, CLOCK = range(5)
POLICY = {"static": STATIC, "lru": LRU, "lfu": LFU, "belady": BELADY, "clock": CLOCK}


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libcachesim.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.moe_cachesim.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_double, vp]
        lib.moe_cachesim.restype = ctypes.c_int64
        _lib = lib
    return _lib


def to_csr(steps):
    """steps[s][l] = iterable of the distinct experts step s needs in layer l ->
    (trace int32, offsets int32 [S*L+1], L)"""
    L = len(steps[0]) if steps else 1
    flat, off = [], [0]
    for st in steps:
        assert len(st) == L
        for ex in st:
            ex = sorted(set(int(e) for e in ex))
            flat.extend(ex)
            off.append(len(flat))
    return np.asarray(flat, np.int32), np.asarray(off, np.int32), L


def simulate(trace, off, L, n_experts, slots, policy, decay=0.995):
    """misses per step (int64 [steps]) of `policy` with `slots` slots per layer"""
    trace = np.ascontiguousarray(trace, np.int32)
    off = np.ascontiguousarray(off, np.int32)
    steps = (len(off) - 1) // L
    pol = POLICY[policy] if isinstance(policy, str) else int(policy)
    misses = np.zeros(max(steps, 1), np.int64)
    tot = _load().moe_cachesim(trace.ctypes.data, off.ctypes.data, steps, L, n_experts, slots,
                               pol, decay, misses.ctypes.data)
    if tot < 0:
        raise ValueError("moe_cachesim: bad arguments")
    return misses[:steps]
