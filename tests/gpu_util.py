"""Helpers of the GPU parity tests: build a layer's inputs on the device, run the
HIP path through the C-ABI, and evaluate the oracle on the same bytes."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from synth.device import DeviceLayer, x_device


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def make_layer_api(cfg, dl: DeviceLayer, max_tokens: int, n_layers: int = 1, layer_slot: int = 0):
    from bit_moe_expert_router_amd import MoELayer
    ml = MoELayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits, cfg.group,
                  cfg.scale_f16, cfg.shared_inter, max_tokens, n_layers, dl.arena.device)
    ml.set_table(layer_slot, dl.refs)
    if dl.shared is not None:
        ml.set_shared(layer_slot, *dl.shared)
    return ml


def run_gpu(cfg, dl: DeviceLayer, x_dev: torch.Tensor, ml=None, layer_slot=0, routing=None):
    """route (unless routing is given) + forward; returns numpy results"""
    T = x_dev.shape[0]
    if ml is None:
        ml = make_layer_api(cfg, dl, max(T, 1))
    if routing is None:
        r = ml.route(x_dev, dl.router, dl.bias)
    else:
        r = routing
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=x_dev.device)
    pair_out = torch.empty((T * cfg.top_k, cfg.hidden), dtype=torch.float32, device=x_dev.device)
    ml.forward(layer_slot, x_dev, r, out, pair_out)
    torch.cuda.synchronize()
    return dict(ids=r.topk_ids.cpu().numpy(), w=r.topk_w.cpu().numpy(),
                offsets=r.expert_offsets.cpu().numpy(), sorted=r.sorted_pairs.cpu().numpy(),
                pos=r.pair_pos.cpu().numpy(), out=out.cpu().numpy(),
                pair_out=pair_out.cpu().numpy(), ml=ml)


class HostExperts:
    """Lazily generated host copies of a layer's expert blobs (logical ids)."""

    def __init__(self, cfg, layer=0):
        self.cfg, self.layer = cfg, layer
        self.off = synth.matrix_offsets(cfg)
        self._cache = {}

    def blobs(self, e):
        if e not in self._cache:
            b = synth.expert_blob(self.cfg, self.layer, e)
            o = self.off
            self._cache[e] = (b[o[0]:o[1]], b[o[1]:o[2]], b[o[2]:])
        return self._cache[e]

    def ffn(self, x_bits_row, e):
        cfg = self.cfg
        xf = synth.bf16_to_f32(x_bits_row).astype(np.float64)
        g, u, d = self.blobs(e)
        return oracle.expert_ffn(xf, g, u, d, cfg.hidden, cfg.inter, cfg.bits, cfg.group,
                                 cfg.scale_f16)

    def ffn_pairs(self, xh, ids, pairs):
        """oracle y(t,k) of the given pairs p = t*K + k ({p: y}); the pairs of one
        expert go through the oracle together (each dequantised row formed once)"""
        cfg = self.cfg
        flat = np.asarray(ids).reshape(-1)
        by_e = {}
        for p in pairs:
            by_e.setdefault(int(flat[p]), []).append(int(p))
        out = {}
        for e, ps in by_e.items():
            X = synth.bf16_to_f32(np.stack([xh[p // cfg.top_k] for p in ps])).astype(np.float64)
            g, u, d = self.blobs(e)
            Y = oracle.expert_ffn_multi(X, g, u, d, cfg.hidden, cfg.inter, cfg.bits, cfg.group,
                                        cfg.scale_f16)
            for p, y in zip(ps, Y):
                out[p] = y
        return out

    def shared(self):
        if not self.cfg.shared_inter:
            return None
        return synth.shared_weights(self.cfg, self.layer)


def rel_err(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))
