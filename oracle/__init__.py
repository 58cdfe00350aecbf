"""Plain fp64 CPU oracle of the routed-MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package.  The product (``bit_moe_expert_router_amd``) never imports,
links or calls it; the two share no code.  The arithmetic lives in ``oracle.c``
(see its header for what is computed and which page passage each step follows);
this module only marshals numpy arrays to it.

Functions whose result is pinned by the CPU tests (``tests/test_oracle_*.py``):
unpacking (bit bijection, pair structure, packer round trip, one-hot probes),
routing (brute force over all subsets, tie-break, closed-form weights), grouping
(brute force, inverse permutation), expert FFN and combine (dense-gating numpy
formulation, closed forms), RMSNorm (closed form), and the layer invariants.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_d = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.orc_set_threads.restype = None
        lib.orc_set_threads.argtypes = [i32]
        lib.orc_max_threads.restype = i32
        lib.orc_max_threads.argtypes = []
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_double.restype = ctypes.c_double
        lib.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_double_to_bf16.restype = ctypes.c_uint16
        lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_matrix_bytes.restype = ctypes.c_int64
        lib.orc_matrix_bytes.argtypes = [i32] * 4
        lib.orc_code.restype = i32
        lib.orc_code.argtypes = [vp] + [i32] * 7
        lib.orc_scale.restype = ctypes.c_double
        lib.orc_scale.argtypes = [vp] + [i32] * 7
        lib.orc_dequant_row.restype = None
        lib.orc_dequant_row.argtypes = [vp] + [i32] * 6 + [vp]
        lib.orc_matvec.restype = None
        lib.orc_matvec.argtypes = [vp] + [i32] * 5 + [vp, vp]
        lib.orc_matvec_bf16.restype = None
        lib.orc_matvec_bf16.argtypes = [vp, i32, i32, vp, vp]
        lib.orc_route.restype = None
        lib.orc_route.argtypes = [i32] * 4 + [vp] * 7
        lib.orc_permute.restype = None
        lib.orc_permute.argtypes = [i32] * 3 + [vp] * 4
        lib.orc_expert_ffn.restype = None
        lib.orc_expert_ffn.argtypes = [i32] * 5 + [vp] * 5
        lib.orc_expert_ffn_multi.restype = None
        lib.orc_expert_ffn_multi.argtypes = [i32] * 5 + [vp] * 3 + [i32, vp, vp]
        lib.orc_shared_ffn.restype = None
        lib.orc_shared_ffn.argtypes = [i32, i32] + [vp] * 5
        lib.orc_moe_layer.restype = None
        lib.orc_moe_layer.argtypes = [i32] * 8 + [vp] * 6 + [i32] + [vp] * 5
        lib.orc_rmsnorm.restype = None
        lib.orc_rmsnorm.argtypes = [i32, vp, ctypes.c_double, vp]
        lib.orc_rmsnorm_bf16.restype = None
        lib.orc_rmsnorm_bf16.argtypes = [i32, i32, vp, ctypes.c_double, vp]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ------------------------------------------------------------------ threads
def set_threads(n: int):
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return _load().orc_max_threads()


# ------------------------------------------------------------------ scalars
def bf16_to_double(b: int) -> float:
    return _load().orc_bf16_to_double(int(b))


def f16_to_double(h: int) -> float:
    return _load().orc_f16_to_double(int(h))


def double_to_bf16(v: float) -> int:
    return _load().orc_double_to_bf16(float(v))


# ------------------------------------------------------------------ format
def matrix_bytes(rows, cols, bits, group) -> int:
    return _load().orc_matrix_bytes(rows, cols, bits, group)


def code(blob, rows, cols, bits, group, n, g, i) -> int:
    blob = _c(blob, np.uint8)
    return _load().orc_code(_p(blob), rows, cols, bits, group, n, g, i)


def scale(blob, rows, cols, bits, group, scale_f16, n, g) -> float:
    blob = _c(blob, np.uint8)
    return _load().orc_scale(_p(blob), rows, cols, bits, group, int(scale_f16), n, g)


def dequant_row(blob, rows, cols, bits, group, scale_f16, n) -> np.ndarray:
    blob = _c(blob, np.uint8)
    out = np.empty(cols, dtype=np.float64)
    _load().orc_dequant_row(_p(blob), rows, cols, bits, group, int(scale_f16), n, _p(out))
    return out


def dequant(blob, rows, cols, bits, group, scale_f16) -> np.ndarray:
    return np.stack([dequant_row(blob, rows, cols, bits, group, scale_f16, n)
                     for n in range(rows)])


def matvec(blob, rows, cols, bits, group, scale_f16, v) -> np.ndarray:
    blob = _c(blob, np.uint8)
    v = _c(v, np.float64)
    y = np.empty(rows, dtype=np.float64)
    _load().orc_matvec(_p(blob), rows, cols, bits, group, int(scale_f16), _p(v), _p(y))
    return y


# ------------------------------------------------------------------ routing
def route(x_bf16, Wr, bias, K):
    """-> ids int32 [T,K], w float64 [T,K], gap float64 [T], logits float64 [T,E]"""
    x_bf16 = _c(x_bf16, np.uint16)
    Wr = _c(Wr, np.float32)
    T, H = x_bf16.shape
    E = Wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    gap = np.empty(T, dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    _load().orc_route(T, H, E, K, _p(x_bf16), _p(Wr), _p(b), _p(ids), _p(w), _p(gap),
                      _p(logits))
    return ids, w, gap, logits


def permute(ids, E):
    """-> offsets [E+1], sorted_pairs [T*K], pair_pos [T*K] (int32)"""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(T * K, dtype=np.int32)
    pp = np.empty(T * K, dtype=np.int32)
    _load().orc_permute(T, K, E, _p(ids), _p(offsets), _p(sp), _p(pp))
    return offsets, sp[:offsets[E]], pp


# ------------------------------------------------------------------ experts
def expert_ffn(x, gate, up, down, H, I, bits, group, scale_f16) -> np.ndarray:
    x = _c(x, np.float64)
    gate, up, down = (_c(a, np.uint8) for a in (gate, up, down))
    y = np.empty(H, dtype=np.float64)
    _load().orc_expert_ffn(H, I, bits, group, int(scale_f16), _p(gate), _p(up), _p(down),
                           _p(x), _p(y))
    return y


def expert_ffn_multi(X, gate, up, down, H, I, bits, group, scale_f16) -> np.ndarray:
    """expert_ffn of every row of X [n, H] (each dequantised row formed once);
    row j equals expert_ffn(X[j], ...) bit for bit"""
    X = _c(X, np.float64).reshape(-1, H)
    gate, up, down = (_c(a, np.uint8) for a in (gate, up, down))
    n = X.shape[0]
    Y = np.empty((n, H), dtype=np.float64)
    if n:
        _load().orc_expert_ffn_multi(H, I, bits, group, int(scale_f16), _p(gate), _p(up),
                                     _p(down), n, _p(X), _p(Y))
    return Y


def shared_ffn(x, sg, su, sd) -> np.ndarray:
    x = _c(x, np.float64)
    sg, su, sd = (_c(a, np.uint16) for a in (sg, su, sd))
    Is, H = sg.shape
    y = np.empty(H, dtype=np.float64)
    _load().orc_shared_ffn(H, Is, _p(sg), _p(su), _p(sd), _p(x), _p(y))
    return y


def moe_layer(x_bf16, ids, w, gate_tab, up_tab, down_tab, I, bits, group, scale_f16,
              shared=None):
    """Routed-MoE layer for given routing.

    gate_tab/up_tab/down_tab: lists (indexed by logical expert id) of uint8 blobs.
    shared: None or (gate [Is,H], up [Is,H], down [H,Is]) bf16 bit patterns.
    -> out float64 [T,H], pair_out float64 [T*K,H] (pair p = t*K + k, unweighted)
    """
    x_bf16 = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, H = x_bf16.shape
    K = ids.shape[1]
    E = len(gate_tab)
    keep = [_c(b, np.uint8) for b in list(gate_tab) + list(up_tab) + list(down_tab)]
    tabs = []
    for j in range(3):
        arr = (ctypes.c_void_p * E)(*[keep[j * E + e].ctypes.data for e in range(E)])
        tabs.append(arr)
    if shared is not None:
        sg, su, sd = (_c(a, np.uint16) for a in shared)
        Is = sg.shape[0]
    else:
        sg = su = sd = None
        Is = 0
    out = np.empty((T, H), dtype=np.float64)
    pair_out = np.empty((T * K, H), dtype=np.float64)
    _load().orc_moe_layer(T, H, I, E, K, bits, group, int(scale_f16), _p(x_bf16), _p(ids), _p(w),
                          ctypes.cast(tabs[0], ctypes.c_void_p),
                          ctypes.cast(tabs[1], ctypes.c_void_p),
                          ctypes.cast(tabs[2], ctypes.c_void_p), Is, _p(sg), _p(su), _p(sd),
                          _p(out), _p(pair_out))
    return out, pair_out


# ------------------------------------------------------------------ stack glue
def rmsnorm(x, eps=1e-6) -> np.ndarray:
    x = _c(x, np.float64)
    r = np.empty_like(x)
    _load().orc_rmsnorm(x.shape[0], _p(x), eps, _p(r))
    return r


def rmsnorm_bf16(x, eps=1e-6) -> np.ndarray:
    x = _c(x, np.float64)
    T, H = x.shape
    out = np.empty((T, H), dtype=np.uint16)
    _load().orc_rmsnorm_bf16(T, H, _p(x), eps, _p(out))
    return out
