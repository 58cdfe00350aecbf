"""moe_stack_layer (one call per stack layer: the normalisation inside the
routing kernels of batches up to 32 tokens, the residual update inside the
combine) against the three-call sequence moe_rmsnorm_bf16 + moe_route +
moe_forward it replaces, on three layers of the 42-layer stack's shape (shared
expert, remapped tables), through the C-ABI: every layer's normalised input,
routing and output, and the final residual, bit for bit, on each routing and
expert path (one-launch routing at 1 and 2 tokens; the small-batch logits at 3
to 32; the normalisation kernel before the matrix-core logits at 40; the
prefill experts at 100), and with 2-bit, 4-bit G128 and 4-bit G32 codes at 4
tokens.  The three-call sequence itself is checked against the oracle layer by
layer in test_gpu_stack.py."""
import numpy as np
import pytest
import torch

import synth
from synth.device import DeviceLayer
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

L = 3
_layers = {}


def _stack(gpu, name="c4"):
    if name not in _layers:
        cfg = synth.CONFIGS[name]
        _layers[name] = [DeviceLayer.generate(cfg, l, gpu) for l in range(L)]
    return _layers[name]


CASES = [("c4", T) for T in (1, 2, 3, 4, 8, 9, 32, 40, 100)] + [("q2", 4), ("q4", 4), ("c1", 4)]


@pytest.mark.parametrize("name,T", CASES)
def test_stack_layer_equals_three_calls(gpu, name, T):
    from bit_moe_expert_router_amd import MoELayer
    from bit_moe_expert_router_amd.layer import stack_forward, stack_forward_fused

    cfg = synth.CONFIGS[name]
    H = cfg.hidden
    say(f"[stack fused] {name} T={T}")
    layers = _stack(gpu, name)
    ml = MoELayer(H, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits, cfg.group, cfg.scale_f16,
                  cfg.shared_inter, T, L, gpu)
    for l, dl in enumerate(layers):
        ml.set_table(l, dl.refs)
        if dl.shared is not None:
            ml.set_shared(l, *dl.shared)
    x0 = torch.from_numpy(synth.normal_f32(T * H, cfg.seed, 50 + T, synth.SYN_X, 1.0)
                          .reshape(T, H)).to(gpu)
    routers = [dl.router for dl in layers]
    biases = [dl.bias for dl in layers]

    def run(fused):
        resid = x0.clone()
        y = torch.empty((T, H), dtype=torch.int16, device=gpu)
        out = torch.empty((T, H), dtype=torch.float32, device=gpu)
        seen = []

        def on_layer(l, y_, r, out_):
            seen.append((y_.clone(), r.topk_ids.clone(), r.topk_w.clone(),
                         r.expert_offsets.clone(), out_.clone()))

        if fused:
            stack_forward_fused(ml, resid, routers, biases, y, out, on_layer=on_layer)
        else:
            stack_forward(ml, resid, None, routers, biases, y, out, on_layer=on_layer)
            resid += out  # the last layer's output (added by the next normalisation otherwise)
        torch.cuda.synchronize()
        return resid, seen

    ra, sa = run(False)
    rb, sb = run(True)
    for l in range(L):
        for name, a, b in zip(("xn", "ids", "w", "offsets", "out"), sa[l], sb[l]):
            assert torch.equal(a, b), (T, l, name)
    assert torch.equal(ra, rb), T
    assert bool(torch.isfinite(rb).all())
    say(f"[stack fused] {name} T={T}: {L} layers bit-identical")
    ml.close()


def test_stack_layer_argument_checks(gpu):
    import bit_moe_expert_router_amd as m
    from bit_moe_expert_router_amd import MoELayer
    cfg = synth.CONFIGS["c4"]
    layers = _stack(gpu)
    ml = MoELayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.bits, cfg.group,
                  cfg.scale_f16, cfg.shared_inter, 4, 1, gpu)
    resid = torch.zeros((4, cfg.hidden), dtype=torch.float32, device=gpu)
    y = torch.empty((4, cfg.hidden), dtype=torch.int16, device=gpu)
    out = torch.empty_like(resid)
    with pytest.raises(m.MoEError) as ei:  # table never set
        ml.stack_layer(0, resid, layers[0].router, layers[0].bias, y, out)
    assert ei.value.status == m.MOE_E_STATE
    ml.set_table(0, layers[0].refs)
    with pytest.raises(m.MoEError) as ei:  # bad eps
        ml.stack_layer(0, resid, layers[0].router, layers[0].bias, y, out, eps=-1.0)
    assert ei.value.status == m.MOE_E_ARG
    ml.close()
