"""Seeded synthetic inputs for the routed-MoE layer (input generation only).

This module is shared by the tests, the bench and the smoke check.  It holds the
workload shapes, the counter-based generator bindings (``synth_core.h``), the
byte geometry of the packed weight format and a packer for structured test
inputs.  It contains none of the layer's arithmetic: no routing, no dequantised
products, no activation, no combine.  Random values the layer consumes are drawn
here and handed to both the HIP path and the oracle as plain bytes.

Workload shapes follow the GLM-5.3-Flash model the pages serve: 288 routed
experts per MoE layer with 8 picked per token (page "GLM-5.3-Flash EXL3 3.05bpw on
1x RTX 3090 -- RAM/NVMe expert tiering", field ``summary``; page "GLM-5.3-Flash EXL3
3.05bpw on 1x RTX PRO 6000 - GPU expert cache, host-RAM streaming", field
``config.expert_cache.layout``), 42 MoE layers, decode batches of at most 8 tokens
and 8,192-token prefill chunks (page "0xSero/glm53-flash-offload", paragraph
"fast mode (G067)").  Hidden size 5120 and expert intermediate size 1536 are not
printed on the pages; they are consistent with the ~9 MiB per expert at ~3 bpw
the pages state (3 * 5120 * 1536 * 3.05 / 8 = 8.99 MB).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# stream fields (synth_core.h)
SYN_CODES = 1
SYN_SCALES = 2
SYN_X = 3
SYN_ROUTER = 4
SYN_BIAS_PERM = 5
SYN_SLOT_PERM = 6
SYN_SHARED = 7

SCALE_LO = 0.01
SCALE_WIDTH = 0.04
# Shared-expert weights: uniform on [-a, a) with the same second moment as a
# routed expert's dequantised weight q*s (q uniform on [-4, 3], s uniform on
# [0.01, 0.05]): E[q^2] = 5.5, E[s^2] = 1.0333e-3, std 0.0754 -> a = std * sqrt(3).
SHARED_A = math.sqrt(5.5 * (0.05 ** 3 - 0.01 ** 3) / (3 * 0.04)) * math.sqrt(3.0)
ZIPF_S = 1.1


def align(n: int, a: int = 256) -> int:
    return (n + a - 1) // a * a


@dataclass(frozen=True)
class MoEConfig:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    tokens: int
    bits: int
    group: int
    scale_f16: bool          # scale dtype: fp16 if True else bf16
    shared_inter: int = 0    # 0: no shared expert
    layers: int = 1
    seed: int = 0
    zipf: bool = True        # Zipf(1.1) router bias; False: no bias
    remap: bool = False      # pointer table maps logical ids to a permutation of slots
    x_sd: float = 1.0
    router_sd: float = 0.02

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# The five workloads.  c1: tiny, checkable on the CPU in seconds.  c2: one
# GLM-shaped layer at decode batch 1.  c3: decode batch 8 with a shared expert and
# a remapped pointer table.  c4: the 42-layer stack at decode batch 4.  c5: an
# 8,192-token prefill chunk.
CONFIGS = {
    "c1": MoEConfig("c1", 256, 128, 16, 2, 4, 4, 32, True, seed=1, zipf=False),
    "c2": MoEConfig("c2", 5120, 1536, 288, 8, 1, 3, 128, False, seed=2),
    "c3": MoEConfig("c3", 5120, 1536, 288, 8, 8, 3, 128, False, shared_inter=1536, seed=3,
                    remap=True),
    "c4": MoEConfig("c4", 5120, 1536, 288, 8, 4, 3, 128, False, shared_inter=1536, layers=42,
                    seed=4, remap=True),
    "c5": MoEConfig("c5", 5120, 1536, 288, 8, 8192, 3, 128, False, seed=5),
    # the same layer with 2-bit and 4-bit codes in groups of 128 (2.125 and 4.125
    # bits per weight; the 2x RTX 5090 page serves a 2.05 bpw quantisation)
    "q2": MoEConfig("q2", 5120, 1536, 288, 8, 1, 2, 128, False, seed=6),
    "q4": MoEConfig("q4", 5120, 1536, 288, 8, 1, 4, 128, False, seed=7),
}


# ---------------------------------------------------------------- format geometry
@dataclass(frozen=True)
class MatrixLayout:
    rows: int
    cols: int
    bits: int
    group: int
    unit_bytes: int      # bytes of one unit (one row, one group)
    n_groups: int
    codes_bytes: int
    scales_off: int
    scales_bytes: int
    nbytes: int


def matrix_layout(rows: int, cols: int, bits: int, group: int) -> MatrixLayout:
    """Byte geometry of one packed matrix (rows = outputs, cols = reduction dim)."""
    if rows % 64 or cols % group or (bits * group) % 128:
        raise ValueError(f"unsupported matrix {rows}x{cols} bits={bits} group={group}")
    unit = bits * group // 8
    ng = cols // group
    codes = (rows // 64) * ng * 64 * unit
    soff = align(codes)
    sbytes = rows * ng * 2
    return MatrixLayout(rows, cols, bits, group, unit, ng, codes, soff, sbytes,
                        soff + align(sbytes))


def expert_layouts(cfg: MoEConfig):
    """(gate, up, down) layouts; gate/up are [inter, hidden], down is [hidden, inter]."""
    g = matrix_layout(cfg.inter, cfg.hidden, cfg.bits, cfg.group)
    d = matrix_layout(cfg.hidden, cfg.inter, cfg.bits, cfg.group)
    return g, g, d


def expert_bytes(cfg: MoEConfig) -> int:
    return sum(l.nbytes for l in expert_layouts(cfg))


def matrix_offsets(cfg: MoEConfig):
    """byte offsets of gate, up, down inside one expert blob"""
    g, u, d = expert_layouts(cfg)
    return 0, g.nbytes, g.nbytes + u.nbytes


def shared_bytes(cfg: MoEConfig) -> int:
    return 3 * cfg.shared_inter * cfg.hidden * 2


# ---------------------------------------------------------------- native binding
_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        lib.syn_stream_key.restype = u64
        lib.syn_stream_key.argtypes = [u64] * 5
        lib.syn_draw_at.restype = u64
        lib.syn_draw_at.argtypes = [u64, u64]
        lib.syn_fill_codes.argtypes = [vp, u64, u64, u64, u64, u64]
        lib.syn_fill_scales.argtypes = [vp, u64, u64, u64, u64, u64, dbl, dbl, ctypes.c_int]
        lib.syn_fill_uniform_bf16.argtypes = [vp, u64, u64, u64, u64, u64, u64, dbl]
        lib.syn_fill_normal_bf16.argtypes = [vp, u64, u64, u64, u64, u64, dbl]
        lib.syn_fill_normal_f32.argtypes = [vp, u64, u64, u64, u64, u64, dbl]
        lib.syn_permutation.argtypes = [vp, i32, u64, u64, u64]
        for f in ("syn_fill_codes", "syn_fill_scales", "syn_fill_uniform_bf16",
                  "syn_fill_normal_bf16", "syn_fill_normal_f32", "syn_permutation"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def stream_key(seed, layer, fld, expert=0, matrix=0) -> int:
    return _load().syn_stream_key(seed, layer, fld, expert, matrix)


def draw(key: int, i: int) -> int:
    return _load().syn_draw_at(key, i)


def codes_bytes(n: int, seed: int, layer: int, expert: int, matrix: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _load().syn_fill_codes(_ptr(out), n, seed, layer, expert, matrix)
    return out


def scales_u16(n: int, seed: int, layer: int, expert: int, matrix: int, f16: bool) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().syn_fill_scales(_ptr(out), n, seed, layer, expert, matrix, SCALE_LO, SCALE_WIDTH,
                            int(f16))
    return out


def normal_bf16(n: int, seed: int, layer: int, fld: int, sd: float, expert: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().syn_fill_normal_bf16(_ptr(out), n, seed, layer, fld, expert, sd)
    return out


def normal_f32(n: int, seed: int, layer: int, fld: int, sd: float, expert: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().syn_fill_normal_f32(_ptr(out), n, seed, layer, fld, expert, sd)
    return out


def uniform_bf16(n: int, seed: int, layer: int, fld: int, expert: int, matrix: int,
                 a: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().syn_fill_uniform_bf16(_ptr(out), n, seed, layer, fld, expert, matrix, a)
    return out


def permutation(n: int, seed: int, layer: int, fld: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().syn_permutation(_ptr(out), n, seed, layer, fld)
    return out


# ---------------------------------------------------------------- layer inputs
def matrix_blob(lay: MatrixLayout, seed: int, layer: int, expert: int, matrix: int,
                f16: bool) -> np.ndarray:
    """One packed matrix blob (codes region, pad, scales region, pad) on the host."""
    blob = np.zeros(lay.nbytes, dtype=np.uint8)
    blob[:lay.codes_bytes] = codes_bytes(lay.codes_bytes, seed, layer, expert, matrix)
    sc = scales_u16(lay.rows * lay.n_groups, seed, layer, expert, matrix, f16)
    blob[lay.scales_off:lay.scales_off + lay.scales_bytes] = sc.view(np.uint8)
    return blob


def expert_blob(cfg: MoEConfig, layer: int, expert: int) -> np.ndarray:
    """gate | up | down blobs of logical expert `expert`, concatenated."""
    parts = [matrix_blob(l, cfg.seed, layer, expert, m, cfg.scale_f16)
             for m, l in enumerate(expert_layouts(cfg))]
    return np.concatenate(parts)


def x_bf16(cfg: MoEConfig, tokens: int | None = None, layer: int = 0) -> np.ndarray:
    t = cfg.tokens if tokens is None else tokens
    return normal_bf16(t * cfg.hidden, cfg.seed, layer, SYN_X, cfg.x_sd).reshape(t, cfg.hidden)


def router_f32(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    return normal_f32(cfg.n_experts * cfg.hidden, cfg.seed, layer, SYN_ROUTER,
                      cfg.router_sd).reshape(cfg.n_experts, cfg.hidden)


def zipf_bias(cfg: MoEConfig, layer: int = 0) -> np.ndarray | None:
    """Per-expert router bias -s*ln(rank), ranks 1..E assigned by a seeded
    permutation, so that exp(bias) follows Zipf(s) over experts."""
    if not cfg.zipf:
        return None
    perm = permutation(cfg.n_experts, cfg.seed, layer, SYN_BIAS_PERM)
    rank = np.empty(cfg.n_experts, dtype=np.float64)
    rank[perm] = np.arange(1, cfg.n_experts + 1, dtype=np.float64)
    return (-ZIPF_S * np.log(rank)).astype(np.float32)


def slot_permutation(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """physical slot of each logical expert (identity when cfg.remap is False)"""
    if not cfg.remap:
        return np.arange(cfg.n_experts, dtype=np.int32)
    return permutation(cfg.n_experts, cfg.seed, layer, SYN_SLOT_PERM)


def shared_weights(cfg: MoEConfig, layer: int = 0):
    """Shared-expert (gate [Is,H], up [Is,H], down [H,Is]) as bf16 bit patterns,
    row-major."""
    if not cfg.shared_inter:
        return None
    I, H = cfg.shared_inter, cfg.hidden
    g = uniform_bf16(I * H, cfg.seed, layer, SYN_SHARED, 0, 0, SHARED_A).reshape(I, H)
    u = uniform_bf16(I * H, cfg.seed, layer, SYN_SHARED, 0, 1, SHARED_A).reshape(I, H)
    d = uniform_bf16(H * I, cfg.seed, layer, SYN_SHARED, 0, 2, SHARED_A).reshape(H, I)
    return g, u, d


# ---------------------------------------------------------------- packer
# Field bit offsets of the five 3-bit fields inside each 16-bit half of a word of
# a 3-bit unit; the sixth position (bit 0 of each half) carries one bit of one of
# the unit's last eight codes.
Q3_FIELD_OFF = (1, 4, 7, 10, 13)


def pack_unit(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the codes (unsigned, < 2**bits) of units into little-endian words.

    codes: [..., G] integer array; returns [..., bits*G/32] uint32.
    """
    codes = np.asarray(codes, dtype=np.uint32)
    G = codes.shape[-1]
    lead = codes.shape[:-1]
    if bits == 4:
        if G not in (32, 128):
            raise ValueError("4-bit units hold 32 or 128 codes")
        w = np.zeros(lead + (G // 8,), dtype=np.uint32)
        for P in range(G // 2):
            d, f = P >> 2, P & 3
            w[..., d] |= (codes[..., 2 * P] & 15) << (4 * f)
            w[..., d] |= (codes[..., 2 * P + 1] & 15) << (16 + 4 * f)
        return w
    if bits == 2:
        if G != 128:
            raise ValueError("2-bit units hold 128 codes")
        w = np.zeros(lead + (8,), dtype=np.uint32)
        for P in range(64):
            d, f = P >> 3, P & 7
            w[..., d] |= (codes[..., 2 * P] & 3) << (2 * f)
            w[..., d] |= (codes[..., 2 * P + 1] & 3) << (16 + 2 * f)
        return w
    if bits == 3:
        if G != 128:
            raise ValueError("3-bit units hold 128 codes")
        w = np.zeros(lead + (12,), dtype=np.uint32)
        for P in range(60):
            d, f = P // 5, P % 5
            o = Q3_FIELD_OFF[f]
            w[..., d] |= (codes[..., 2 * P] & 7) << o
            w[..., d] |= (codes[..., 2 * P + 1] & 7) << (16 + o)
        for m in range(4):
            P = 60 + m
            for b in range(3):
                w[..., 3 * m + b] |= ((codes[..., 2 * P] >> b) & 1) << 0
                w[..., 3 * m + b] |= ((codes[..., 2 * P + 1] >> b) & 1) << 16
        return w
    raise ValueError(f"unsupported bits {bits}")


def pack_matrix(codes: np.ndarray, scales_u16: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Pack a [N, Kd] matrix of unsigned codes and [N, Kd/G] 16-bit scale bit
    patterns into one blob of the packed format."""
    N, Kd = codes.shape
    lay = matrix_layout(N, Kd, bits, group)
    ng = lay.n_groups
    units = codes.reshape(N // 64, 64, ng, group).transpose(0, 2, 1, 3)  # [rb, g, lane, G]
    words = pack_unit(units, bits)                                       # [rb, g, lane, W]
    C = lay.unit_bytes // 16
    # chunk j of tile (rb, g) holds words 4j..4j+3 of every lane, lane-major
    words = words.reshape(N // 64, ng, 64, C, 4).transpose(0, 1, 3, 2, 4)
    blob = np.zeros(lay.nbytes, dtype=np.uint8)
    blob[:lay.codes_bytes] = np.ascontiguousarray(words).view(np.uint8).reshape(-1)
    # scales in tile order: tile (rb, g) holds the scales of its 64 rows
    sc = np.asarray(scales_u16, dtype=np.uint16).reshape(N // 64, 64, ng).transpose(0, 2, 1)
    blob[lay.scales_off:lay.scales_off + lay.scales_bytes] = np.ascontiguousarray(sc).view(np.uint8).reshape(-1)
    return blob


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float array -> bfloat16 bit patterns (RNE via binary32)."""
    f = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).view(np.uint16)
