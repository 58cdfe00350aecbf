"""Device-side placement of the seeded synthetic inputs (input generation only).

Large weight stacks are generated directly in device memory by the fill kernels
of libsynth_dev.so, which evaluate the same counter-based definitions as the
host generator, so every byte equals what ``synth.expert_blob`` would produce on
the host.  Small inputs (activations, router, bias) are generated on the host and
uploaded.  Nothing here computes any part of the MoE layer.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
import torch

from . import (SCALE_LO, SCALE_WIDTH, SHARED_A, SYN_SHARED, MoEConfig, expert_bytes,
               expert_layouts, matrix_offsets, router_f32, slot_permutation, x_bf16, zipf_bias,
               shared_weights)

_HERE = os.path.dirname(os.path.abspath(__file__))
_dev = None


def _load_dev():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u64, vp, dbl, i = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        lib.syn_dev_fill_codes.argtypes = [vp, u64, u64, u64, u64, u64, vp]
        lib.syn_dev_fill_scales.argtypes = [vp, u64, u64, u64, u64, u64, dbl, dbl, i, vp]
        lib.syn_dev_fill_uniform_bf16.argtypes = [vp, u64, u64, u64, u64, u64, u64, dbl, vp]
        for f in ("syn_dev_fill_codes", "syn_dev_fill_scales", "syn_dev_fill_uniform_bf16"):
            getattr(lib, f).restype = ctypes.c_int
        _dev = lib
    return _dev


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


def fill_expert(dst_ptr: int, cfg: MoEConfig, layer: int, expert: int, stream: int):
    """Write logical expert `expert` of `layer` (gate | up | down) at dst_ptr."""
    lib = _load_dev()
    for m, (lay, off) in enumerate(zip(expert_layouts(cfg), matrix_offsets(cfg))):
        _ok(lib.syn_dev_fill_codes(dst_ptr + off, lay.codes_bytes, cfg.seed, layer, expert, m,
                                   stream), "fill codes")
        _ok(lib.syn_dev_fill_scales(dst_ptr + off + lay.scales_off, lay.rows * lay.n_groups,
                                    cfg.seed, layer, expert, m, SCALE_LO, SCALE_WIDTH,
                                    int(cfg.scale_f16), stream), "fill scales")


@dataclass
class DeviceLayer:
    cfg: MoEConfig
    layer: int
    arena: torch.Tensor                  # uint8 [E * expert_bytes]: slot s at s * expert_bytes
    slots: np.ndarray                    # physical slot of each logical expert
    refs: List[Tuple[int, int, int]]     # per logical expert: gate, up, down addresses
    router: torch.Tensor                 # fp32 [E, H]
    bias: Optional[torch.Tensor]         # fp32 [E] or None
    shared: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]

    @staticmethod
    def generate(cfg: MoEConfig, layer: int, device, slots: Optional[np.ndarray] = None,
                 on_device: bool = True) -> "DeviceLayer":
        device = torch.device(device)
        eb = expert_bytes(cfg)
        E = cfg.n_experts
        if slots is None:
            slots = slot_permutation(cfg, layer)
        arena = torch.empty(E * eb, dtype=torch.uint8, device=device)
        base = arena.data_ptr()
        if on_device:
            stream = torch.cuda.current_stream(device).cuda_stream
            for e in range(E):
                fill_expert(base + int(slots[e]) * eb, cfg, layer, e, stream)
        else:
            from . import expert_blob
            host = np.empty(E * eb, dtype=np.uint8)
            for e in range(E):
                s = int(slots[e])
                host[s * eb:(s + 1) * eb] = expert_blob(cfg, layer, e)
            arena.copy_(torch.from_numpy(host))
        off = matrix_offsets(cfg)
        refs = [tuple(base + int(slots[e]) * eb + o for o in off) for e in range(E)]
        router = torch.from_numpy(router_f32(cfg, layer)).to(device)
        b = zipf_bias(cfg, layer)
        bias = None if b is None else torch.from_numpy(b).to(device)
        shared = None
        if cfg.shared_inter and on_device:
            I, H = cfg.shared_inter, cfg.hidden
            shared = (torch.empty((I, H), dtype=torch.int16, device=device),
                      torch.empty((I, H), dtype=torch.int16, device=device),
                      torch.empty((H, I), dtype=torch.int16, device=device))
            stream = torch.cuda.current_stream(device).cuda_stream
            for m, t in enumerate(shared):
                _ok(_load_dev().syn_dev_fill_uniform_bf16(t.data_ptr(), t.numel(), cfg.seed,
                                                          layer, SYN_SHARED, 0, m, SHARED_A,
                                                          stream), "fill shared")
        elif cfg.shared_inter:
            shared = tuple(torch.from_numpy(a.view(np.int16)).to(device)
                           for a in shared_weights(cfg, layer))
        return DeviceLayer(cfg, layer, arena, np.asarray(slots), refs, router, bias, shared)

    def expert_host(self, e: int) -> np.ndarray:
        """bytes of logical expert e read back from the device (for checking the
        device fill against the host generator)"""
        eb = expert_bytes(self.cfg)
        s = int(self.slots[e])
        return self.arena[s * eb:(s + 1) * eb].cpu().numpy()


def x_device(cfg: MoEConfig, device, tokens=None, layer=0) -> Tuple[np.ndarray, torch.Tensor]:
    """activations: host bf16 bits [T, H] and the same bytes on the device"""
    xh = x_bf16(cfg, tokens, layer)
    return xh, torch.from_numpy(xh.view(np.int16)).to(device)
