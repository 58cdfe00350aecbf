"""moe_forward_noalloc (for callers that cannot allocate) against moe_forward,
through the C-ABI: the same kernels, so the outputs must be bit-identical, on
two calls in a row, the second with a smaller batch; and a batch too large for
the library's scratch is refused with a message."""
import numpy as np
import pytest
import torch

import synth
from synth.device import DeviceLayer, x_device
from tests.gpu_util import make_layer_api, say

pytestmark = pytest.mark.gpu


def _run_both(ml, dl, cfg, T, gpu):
    import bit_moe_expert_router_amd as m
    _, xd = x_device(cfg, gpu, tokens=T)
    r = ml.route(xd, dl.router, dl.bias)
    out_ref = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    po_ref = torch.empty((T * cfg.top_k, cfg.hidden), dtype=torch.float32, device=gpu)
    ml.forward(0, xd, r, out_ref, po_ref)
    out = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device=gpu)
    po = torch.full((T * cfg.top_k, cfg.hidden), float("nan"), dtype=torch.float32, device=gpu)
    m.moe_forward_noalloc(ml.ctx, 0, xd, T, r.topk_ids, r.topk_w, r.expert_offsets,
                          r.sorted_pairs, out, po)
    torch.cuda.synchronize()
    return out, po, out_ref, po_ref


@pytest.mark.parametrize("name,Ts", [("c3", (8, 2)), ("c2", (2, 1)), ("c3", (15, 5))])
def test_noalloc_matches_forward(gpu, name, Ts):
    cfg = synth.CONFIGS[name]
    say(f"[noalloc] {name} T={Ts}")
    dl = DeviceLayer.generate(cfg, 0, gpu)
    ml = make_layer_api(cfg, dl, max(Ts))
    for T in Ts:  # two calls in a row, the second smaller
        out, po, out_ref, po_ref = _run_both(ml, dl, cfg, T, gpu)
        assert torch.equal(out, out_ref), (name, T)
        assert torch.equal(po, po_ref), (name, T)
    ml.close()


def test_noalloc_refuses_too_large(gpu):
    import bit_moe_expert_router_amd as m
    cfg = synth.CONFIGS["c3"]
    say("[noalloc] too large")
    dl = DeviceLayer.generate(cfg, 0, gpu)
    T = 16
    ml = make_layer_api(cfg, dl, T)
    _, xd = x_device(cfg, gpu, tokens=T)
    r = ml.route(xd, dl.router, dl.bias)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=gpu)
    with pytest.raises(m.MoEError) as ei:
        m.moe_forward_noalloc(ml.ctx, 0, xd, T, r.topk_ids, r.topk_w, r.expert_offsets,
                              r.sorted_pairs, out, None)
    assert ei.value.status == m.MOE_E_ARG and "scratch" in str(ei.value)
    ml.close()
