"""Routing and the activation quantisation in one launch
(moe_route_topk_quantize, then the FFN with x_quantized): the layer's output,
ids and weights are bit-identical to routing alone followed by the FFN that
quantises x itself, for E4M3 and MXFP4 weights, top-k with a shared expert,
top-1 (FFN and combine in one call), grouped sigmoid routing, and the
one-stage schedule; two layers in a row on one workspace each use their own x."""
import numpy as np
import pytest
import torch

import moe_synth as ms
from gpu_helpers import device, make_gpu_layer, say

pytestmark = pytest.mark.gpu


def both(cfg, L, B=None, schedule="two_launch"):
    fused = make_gpu_layer(cfg, L, B, schedule=schedule)
    assert fused.route_quant, "E4M3 / MXFP4 layers route and quantise in one launch"
    out_f = fused.forward(L["x"], L["logits"], L["bias"]).clone()
    ids_f, w_f = fused.topk_ids.clone(), fused.topk_weights.clone()
    plain = make_gpu_layer(cfg, L, B, schedule=schedule)
    plain.route_quant = False
    out_p = plain.forward(L["x"], L["logits"], L["bias"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(ids_f, plain.topk_ids)
    assert torch.equal(w_f.view(torch.int32), plain.topk_weights.view(torch.int32))
    assert torch.equal(out_f.view(torch.int16), out_p.view(torch.int16))
    return fused, out_f


@pytest.mark.parametrize("name,over", [
    ("prefill_fp8", dict(T=333, H=768, I=256, E=12)),                       # top-1 + shared expert
    ("prefill_fp4", dict(T=333, H=768, I=384, E=12)),                       # top-1: one call
    ("decode_fp4", dict(T=96, H=512, I=256, E=16, K=4, n_group=4, topk_group=2)),
    ("prefill_fp8_512", dict(T=256, H=512, I=256, E=16, K=4)),
])
def test_route_quantize_matches_separate_quantisation(name, over):
    dev = device()
    cfg = ms.scaled(name, **over)
    L = ms.make_layer(cfg, device=dev)
    for B in (32, 128):
        layer, _ = both(cfg, L, B)
        say(f"{name} B={B}: route + quantise in one launch bit-identical (top1={layer.top1})")


def test_route_quantize_one_stage_schedule():
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=200, H=512, I=256, E=8)
    L = ms.make_layer(cfg, device=dev)
    layer, _ = both(cfg, L, 64, schedule="fused")
    assert layer.fused_status() == 0


def test_route_quantize_layers_in_a_row_use_their_own_x():
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=300, H=512, I=256, E=8)
    L0 = ms.make_layer(cfg, device=dev, seed=0)
    L1 = ms.make_layer(cfg, device=dev, seed=1, weights=False)
    layer = make_gpu_layer(cfg, L0, 64)
    ref = make_gpu_layer(cfg, L0, 64)
    ref.route_quant = False
    for Lx in (L0, L1, L0):
        got = layer.forward(Lx["x"], Lx["logits"], L0["bias"]).clone()
        want = ref.forward(Lx["x"], Lx["logits"], L0["bias"]).clone()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    say("three layers in a row on one workspace: each quantised its own x")
