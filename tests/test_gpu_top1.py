"""The FFN and the combine of a top-1 layer as one call (moe_grouped_ffn_top1)
on the GPU: it must give the same output bits as moe_grouped_ffn followed by
moe_combine (which the layer tests compare with the oracle), zero rows for
tokens whose id is outside [0,E), and leave the backward unchanged."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import routing_align_sort_amd as moe
from gpu_helpers import (as_library_weights, compare_out, device, make_gpu_layer, oracle_layer_cached,
                         say)

pytestmark = pytest.mark.gpu


def small_cfg(name):
    over = dict(T=300, H=256, I=256, E=8)
    if name == "prefill_fp8":
        over.update(shared=False)
    return ms.scaled(name, **over)


def top1_vs_separate(cfg, B, out_dtype, p_skip, seed):
    """moe_grouped_ffn_top1 against moe_grouped_ffn + moe_combine on ids with a
    share p_skip of out-of-range tokens (canonical and packed weights)."""
    dev = device()
    L = ms.make_layer(cfg, device=dev)
    w13, w2, s13, s2 = as_library_weights(L)
    T, E = cfg["T"], cfg["E"]
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, (T, 1)).astype(np.int32)
    bad = rng.random(T) < p_skip
    ids[bad, 0] = rng.choice([-1, E, E + 5], size=int(bad.sum()))
    tid = torch.tensor(ids, device=dev)
    w = torch.tensor(rng.random((T, 1)).astype(np.float32) + 0.25, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    srt, eids, ntpp = al["sorted_token_ids"], al["expert_ids"], al["num_tokens_post_padded"]
    for packed in (False, True):
        a13, a2, b13, b2 = w13, w2, s13, s2
        if packed:
            a13, a2 = moe.moe_prepack_weights(w13, w2)
            if w13.dtype == moe.FP4:
                b13, b2 = moe.moe_prepack_block_scales(s13, s2, cfg["H"], cfg["I"])
        y = moe.moe_grouped_ffn(L["x"], a13, a2, srt, eids, ntpp, K=1, B=B, w13_scale=b13, w2_scale=b2,
                                packed=packed)
        ref = moe.moe_combine(y, w, tid, E, out_dtype=out_dtype)
        out = torch.full((T, cfg["H"]), float("nan"), dtype=out_dtype, device=dev)
        got = moe.moe_grouped_ffn_top1(L["x"], a13, a2, srt, eids, ntpp, tid, w, B=B, w13_scale=b13,
                                       w2_scale=b2, out_dtype=out_dtype, out=out, packed=packed)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"packed={packed}"
        assert (got[torch.tensor(bad, device=dev)] == 0).all()
    say(f"  {int(bad.sum())} of {T} skipped tokens zeroed; bit-identical to FFN + combine (canonical and packed)")


@pytest.mark.parametrize("name", ["prefill_bf16", "prefill_fp8", "prefill_fp4"])
@pytest.mark.parametrize("B", [16, 64, 128])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_top1_equals_ffn_then_combine(name, B, out_dtype):
    say(f"top-1 {name} B={B} out {out_dtype}")
    top1_vs_separate(small_cfg(name), B, out_dtype, 0.1, B)


@pytest.mark.parametrize("p_skip", [0.5, 0.9])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_top1_mostly_skipped_tokens_full_width(p_skip, out_dtype):
    # an expert-parallel share: most tokens are handled by other experts'
    # owners, so their ids are out of range and their rows are zeroed here,
    # at the full hidden width
    say(f"top-1 with {p_skip:.0%} skipped tokens, H 7168, out {out_dtype}")
    cfg = ms.scaled("prefill_bf16", T=1500, H=7168, I=256, E=8)
    top1_vs_separate(cfg, 64, out_dtype, p_skip, int(p_skip * 100))


def test_top1_layer_full_size_prefill_bf16():
    dev = device()
    cfg = ms.CONFIGS["prefill_bf16"]
    say("generating prefill bf16 weights (32 experts, 2.8 GB)")
    L = ms.make_layer(cfg, device=dev)
    one = make_gpu_layer(cfg, L)
    two = make_gpu_layer(cfg, L, top1=False)
    assert one.top1 and not two.top1
    a = one.forward(L["x"], L["logits"], L["bias"]).clone()
    b = two.forward(L["x"], L["logits"], L["bias"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    say("prefill bf16, B 64: the top-1 layer equals FFN + combine bit for bit")
    ids, w, toks, ref, _ = oracle_layer_cached("prefill_bf16", cfg, L)
    compare_out(a, toks, ref, cfg["dtype"], "prefill bf16 top-1, B 64")


def test_backward_after_a_top1_forward():
    # the top-1 forward writes no slot rows; the backward recomputes them
    dev = device()
    cfg = ms.scaled("prefill_bf16", T=256, H=256, I=256, E=8)
    L = ms.make_layer(cfg, device=dev)
    d_out = torch.tensor(np.random.default_rng(1).standard_normal((cfg["T"], cfg["H"])).astype(np.float32),
                         device=dev)
    res = []
    for top1 in ("auto", False):
        layer = make_gpu_layer(cfg, L, top1=top1)
        layer.forward(L["x"], L["logits"], L["bias"])
        res.append([t.clone() for t in layer.backward(L["x"], L["logits"], d_out)])
        torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)
    say("backward after a top-1 forward equals the backward after FFN + combine")
