"""Convenience holder around the C-ABI: one context, its workspace and the
routing buffers, for one or more layers of the same shape.  Marshalling only."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (moe_create, moe_destroy, moe_forward, moe_rmsnorm_bf16, moe_route,
               moe_set_shared, moe_workspace_bytes, moe_workspace_init, set_expert_table)


@dataclass
class RoutingBuffers:
    topk_ids: torch.Tensor        # int32 [T, K]
    topk_w: torch.Tensor          # fp32 [T, K]
    expert_offsets: torch.Tensor  # int32 [E+1]
    sorted_pairs: torch.Tensor    # int32 [T*K]
    pair_pos: torch.Tensor        # int32 [T*K]


class MoELayer:
    """Routed-MoE layers of one shape on one device.

    experts: per layer, a sequence of E (gate, up, down) device addresses in
    logical order.  shared: per layer, None or (gate, up, down) bf16 tensors.
    """

    def __init__(self, hidden, inter, n_experts, top_k, bits, group, scale_f16, shared_inter,
                 max_tokens, n_layers=1, device="cuda"):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.max_tokens = max_tokens
        self.device = torch.device(device)
        self.ctx = moe_create(hidden, inter, n_experts, top_k, bits, group, scale_f16,
                              shared_inter, max_tokens, n_layers)
        nbytes = moe_workspace_bytes(self.ctx, max_tokens)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        moe_workspace_init(self.ctx, self.ws)
        T, K, E = max_tokens, top_k, n_experts
        i32 = dict(dtype=torch.int32, device=self.device)
        self.rb = RoutingBuffers(torch.empty((T, K), **i32),
                                 torch.empty((T, K), dtype=torch.float32, device=self.device),
                                 torch.empty(E + 1, **i32), torch.empty(T * K, **i32),
                                 torch.empty(T * K, **i32))

    def close(self):
        if self.ctx:
            moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_table(self, layer, refs, stream=None):
        set_expert_table(self.ctx, layer, refs, stream)

    def set_shared(self, layer, gate, up, down):
        moe_set_shared(self.ctx, layer, gate, up, down)

    def routing(self, T) -> RoutingBuffers:
        rb = self.rb
        return RoutingBuffers(rb.topk_ids[:T], rb.topk_w[:T], rb.expert_offsets,
                              rb.sorted_pairs[:T * self.top_k], rb.pair_pos[:T * self.top_k])

    def route(self, x_bf16, w_router, bias=None, stream=None) -> RoutingBuffers:
        T = x_bf16.shape[0]
        r = self.routing(T)
        moe_route(self.ctx, x_bf16, T, w_router, bias, r.topk_ids, r.topk_w, r.expert_offsets,
                  r.sorted_pairs, r.pair_pos, self.ws, stream)
        return r

    def forward(self, layer, x_bf16, r: RoutingBuffers, out, pair_out=None, stream=None):
        T = x_bf16.shape[0]
        moe_forward(self.ctx, layer, x_bf16, T, r.topk_ids, r.topk_w, r.expert_offsets,
                    r.sorted_pairs, out, pair_out, self.ws, stream)
        return out

    def layer_forward(self, layer, x_bf16, w_router, bias, out, pair_out=None,
                      stream=None) -> RoutingBuffers:
        """routing + experts + combine of one layer in one library call; returns the routing"""
        from . import moe_layer_forward
        T = x_bf16.shape[0]
        r = self.routing(T)
        moe_layer_forward(self.ctx, layer, x_bf16, T, w_router, bias, r.topk_ids, r.topk_w,
                          r.expert_offsets, r.sorted_pairs, r.pair_pos, out, pair_out, self.ws,
                          stream)
        return r

    def error_word(self) -> int:
        """the workspace's error word (waits for the device)"""
        from . import MOE_WS_ERROR_OFFSET
        return int(self.ws[MOE_WS_ERROR_OFFSET:MOE_WS_ERROR_OFFSET + 4].view(torch.int32).item())

    def clear_error(self):
        from . import MOE_WS_ERROR_OFFSET
        self.ws[MOE_WS_ERROR_OFFSET:MOE_WS_ERROR_OFFSET + 4].zero_()

    def rmsnorm_bf16(self, resid, add, y_bf16, eps=1e-6, stream=None):
        moe_rmsnorm_bf16(self.ctx, resid, add, resid.shape[0], eps, y_bf16, stream)
        return y_bf16

    def stack_layer(self, layer, resid, w_router, bias, xn_bf16, out, eps=1e-6, stream=None):
        """resid += MoE_layer(bf16(RMSNorm(resid))) in one library call; returns the routing"""
        from . import moe_stack_layer
        T = resid.shape[0]
        r = self.routing(T)
        moe_stack_layer(self.ctx, layer, resid, T, eps, w_router, bias, r.topk_ids, r.topk_w,
                        r.expert_offsets, r.sorted_pairs, r.pair_pos, xn_bf16, out, self.ws,
                        stream)
        return r


def stack_forward(ml: MoELayer, resid, add, routers, biases, y, out, on_layer=None, stream=None):
    """One pass of a stack of MoE layers on the residual stream:
    x <- x + MoE_l(bf16(RMSNorm(x))) for l = 0 .. L-1.

    resid: fp32 [T, H], updated in place; add: fp32 [T, H] or None, the output
    still to be added to resid before the first layer (the previous pass's last
    layer).  Each layer's output lands in `out` and is added to resid by the next
    layer's normalisation, so after the pass resid + out is the stack's output.
    y: bf16 [T, H] scratch for the normalised layer input.  on_layer(l, y, r,
    out) is called after layer l is enqueued.
    """
    for l in range(len(routers)):
        ml.rmsnorm_bf16(resid, add if l == 0 else out, y, stream=stream)
        r = ml.route(y, routers[l], biases[l], stream=stream)
        ml.forward(l, y, r, out, stream=stream)
        if on_layer is not None:
            on_layer(l, y, r, out)
    return resid, out


def stack_forward_fused(ml: MoELayer, resid, routers, biases, y, out, on_layer=None, stream=None):
    """The same stack pass with one moe_stack_layer call per layer: resid is
    updated in place to the stack's output (x <- x + MoE_l(bf16(RMSNorm(x)))
    for every layer); y and out hold the last layer's normalised input and
    output.  on_layer(l, y, r, out) is called after layer l is enqueued."""
    for l in range(len(routers)):
        r = ml.stack_layer(l, resid, routers[l], biases[l], y, out, stream=stream)
        if on_layer is not None:
            on_layer(l, y, r, out)
    return resid
