"""The one-stage schedule (both GEMMs in one persistent launch, down tiles
starting as their block's intermediate completes) against the two-launch
schedule: the same operands in the same order, so the results must be the
same bits, every bounded wait must have been satisfied (status word 0), and
the counters must reset between calls.  Also against the oracle."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import routing_align_sort_amd as moe
from gpu_helpers import (TOL, as_library_weights, compare_out, compare_slots, device, oracle_layer_cached,
                         oracle_tokens, rel_err, route_oracle, say, seeded_subset)

pytestmark = pytest.mark.gpu


def layer_for(cfg, L, B, **kw):
    w13, w2, s13, s2 = as_library_weights(L)
    return moe.MoELayer(w13, w2, T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"], n_group=cfg["n_group"],
                        topk_group=cfg["topk_group"], renormalize=cfg["renormalize"],
                        shared=bool(cfg.get("shared")), w13_scale=s13, w2_scale=s2, x_dtype=L["x"].dtype,
                        out_dtype=torch.bfloat16, **kw)


def compare(cfg, L, B, rows="by_token", calls=2):
    two = layer_for(cfg, L, B, rows=rows, top1=False)      # its slot rows are compared
    one = layer_for(cfg, L, B, rows=rows, schedule="fused")
    ref = two.forward(L["x"], L["logits"], L["bias"]).clone()
    for c in range(calls):
        one.y_slots.zero_()
        out = one.forward(L["x"], L["logits"], L["bias"])
        torch.cuda.synchronize()
        assert one.fused_status() == 0, f"a wait gave up (call {c})"
        if rows == "sorted":             # rows holding no slot are not written
            placed = one.sorted < one.T * one.KO
            assert torch.equal(one.y_slots[placed], two.y_slots[placed]), f"y differs (call {c})"
        else:
            assert torch.equal(one.y_slots, two.y_slots), f"y differs (call {c})"
        assert torch.equal(out, ref), f"out differs (call {c})"
    return one, ref


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8", "prefill_fp4"])
@pytest.mark.parametrize("B", [16, 32, 64, 128, 256])
def test_fused_equals_two_launch_small(name, B):
    dev = device()
    if name == "decode_bf16":
        cfg = ms.scaled(name, T=300, H=512, I=384, E=16, K=4, n_group=4, topk_group=2)
    else:
        cfg = ms.scaled(name, T=333, H=768, I=256, E=12)
    L = ms.make_layer(cfg, device=dev)
    _, out = compare(cfg, L, B)
    ids, w = route_oracle(cfg, L)
    ref, _ = oracle_tokens(L["x"], L["w13"], L["w2"], ids, w, np.arange(cfg["T"]), L.get("w13_scale"),
                           L.get("w2_scale"))
    err = rel_err(out.float().cpu().numpy(), ref)
    say(f"fused {name} B={B}: bit-identical to two launches, rel err {err:.3e}")
    assert err <= TOL[cfg["dtype"]]


def test_fused_with_sorted_rows():
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=201, H=512, I=384, E=9)
    L = ms.make_layer(cfg, device=dev)
    for B in (16, 64):
        compare(cfg, L, B, rows="sorted")


def test_fused_single_block_and_empty_experts():
    dev = device()
    # one token, one expert: a single M block, one queue holds everything
    cfg = ms.scaled("decode_bf16", T=1, H=256, I=128, E=8, K=1, n_group=1, topk_group=1)
    L = ms.make_layer(cfg, device=dev)
    compare(cfg, L, 16, calls=3)


@pytest.mark.parametrize("name,B", [("prefill_bf16", 64), ("prefill_fp8", 64), ("decode_bf16", 16),
                                    ("prefill_bf16_512", 128), ("decode_fp4", 16)])
def test_fused_equals_two_launch_full_size(name, B):
    dev = device()
    cfg = ms.CONFIGS[name]
    L = ms.make_layer(cfg, device=dev)
    one, out = compare(cfg, L, B)
    say(f"fused {name} B={B} full size: bit-identical to two launches")
    # and against the oracle directly: every token, or the compute-bound
    # shape's seeded 256-token subset (the layer tests' subset)
    toks = seeded_subset(cfg["T"], 256, 5) if name.endswith("_512") else None
    ids, w, toks, ref, yref = oracle_layer_cached(name, cfg, L, toks)
    compare_out(out, toks, ref, cfg["dtype"], f"fused {name} B={B}")
    compare_slots(one.y_slots, toks, ids, yref, cfg["dtype"], f"fused {name} B={B}")
    del L
    torch.cuda.empty_cache()


def test_fused_graph_replays():
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=160, H=512, I=256, E=8)
    L = ms.make_layer(cfg, device=dev)
    layer = layer_for(cfg, L, 32, schedule="fused")
    want = layer.forward(L["x"], L["logits"], L["bias"]).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(L["x"], L["logits"], L["bias"])
    torch.cuda.synchronize()
    for rep in range(4):
        layer.out.zero_()
        layer.y_slots.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert layer.fused_status() == 0
        assert torch.equal(layer.out, want), rep
        junk = torch.randn(1 << 20, device=dev)
        float(junk.sum().item())
    del g
