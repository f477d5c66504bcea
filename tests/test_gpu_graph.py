"""The whole layer (route -> align -> grouped FFN -> combine) captured in one
HIP graph and replayed: the library never reads device memory on the host,
never allocates and never synchronises, so a captured layer must give the
eager result bit for bit on every replay, also after new inputs are written
into the captured buffers.  Between replays the test runs eager work of its
own and clears the outputs, so a replay that skipped work would be caught."""
import numpy as np
import pytest
import torch

import moe_synth as ms
from gpu_helpers import device, make_gpu_layer, say

pytestmark = pytest.mark.gpu


def eager(layer, x, logits, bias):
    out = layer.forward(x, logits, bias).clone()
    torch.cuda.synchronize()
    return out, layer.y_slots.clone(), layer.sorted.clone()


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8", "prefill_bf16", "prefill_fp4"])
def test_layer_graph_replays_match_eager(name):
    # prefill_bf16 and prefill_fp4 are top-1: their FFN and combine run as one
    # call, with no slot rows; the fp8 and MXFP4 layers route and quantise x
    # in one launch
    dev = device()
    if name == "decode_bf16":
        cfg = ms.scaled(name, T=96, H=512, I=256, E=16, K=4, n_group=4, topk_group=2)
    else:
        cfg = ms.scaled(name, T=160, H=512, I=256, E=8)
    L = ms.make_layer(cfg, device=dev)
    L2 = ms.make_layer(cfg, device=dev, seed=1, weights=False)   # second input set
    layer = make_gpu_layer(cfg, L)
    x = L["x"].clone()
    logits = L["logits"].clone()
    bias = None if L["bias"] is None else L["bias"].clone()

    ref1 = eager(layer, x, logits, bias)                  # also warms every kernel up
    x2, logits2 = L2["x"], L2["logits"]
    x.copy_(x2)
    logits.copy_(logits2)
    ref2 = eager(layer, x, logits, bias)
    assert not torch.equal(ref1[0], ref2[0])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, logits, bias)
    torch.cuda.synchronize()

    for rep in range(4):
        use2 = rep % 2 == 1
        x.copy_(x2 if use2 else L["x"])
        logits.copy_(logits2 if use2 else L["logits"])
        layer.out.zero_()
        layer.y_slots.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = ref2 if use2 else ref1
        say(f"{name}: replay {rep} ({'second' if use2 else 'first'} inputs)")
        assert torch.equal(layer.sorted, want[2]), rep
        if not layer.top1:
            assert torch.equal(layer.y_slots, want[1]), rep
        assert torch.equal(layer.out, want[0]), rep
        # eager work of the program's own between replays
        junk = torch.randn(1 << 20, device=dev)
        float(junk.sum().item())
    del g
    torch.cuda.synchronize()
    assert np.isfinite(ref1[0].float().cpu().numpy()).all()
