"""bf16 slot rows between the grouped FFN and the combine (moe_ffn_params_t's
y_dtype, moe_combine_slots).  Each slot row must be the fp32 path's row
rounded to nearest even, bit for bit; the combine over them must match a
float64 sum of the same bf16 values; and the layer output and the slot rows
stay within the dtype's tolerance of the oracle (every token at the small
shapes and at the prefill fp8 shape, a seeded 256-token subset at 512 tokens
per expert)."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import routing_align_sort_amd as moe
from gpu_helpers import (TOL, compare_out, compare_slots, device, make_gpu_layer, oracle_layer_cached,
                         say, seeded_subset)

pytestmark = pytest.mark.gpu


def forward(cfg, L, B, slot_dtype, schedule="two_launch"):
    layer = make_gpu_layer(cfg, L, B, top1=False, slot_dtype=slot_dtype, schedule=schedule)
    out = layer.forward(L["x"], L["logits"], L["bias"]).clone()
    torch.cuda.synchronize()
    return layer, out


def placed_slots(layer):
    ids = layer.topk_ids.cpu().numpy().ravel()
    return torch.as_tensor(np.flatnonzero((ids >= 0) & (ids < layer.E_slabs)), device=layer.y_slots.device)


def check_rounding_and_combine(l32, l16, label):
    rows = placed_slots(l32)
    y32 = l32.y_slots[rows]
    y16 = l16.y_slots[rows]
    assert y16.dtype == torch.bfloat16
    same = torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
    assert same, f"{label}: bf16 slot rows are not the fp32 rows rounded to nearest even"
    # the combine over the bf16 rows against a float64 sum of the same values
    out32 = moe.moe_combine(l16.y_slots, l16.topk_weights, l16.topk_ids, l16.E_slabs, out_dtype=torch.float32)
    T, K = l16.topk_ids.shape
    ids = l16.topk_ids.cpu().numpy()
    w = l16.topk_weights.cpu().numpy().astype(np.float64)
    keep = ((ids >= 0) & (ids < l16.E_slabs)).astype(np.float64)
    # rows of skipped slots are never written: only placed rows are read
    yk = torch.zeros(T * K, l16.y_slots.shape[-1], dtype=torch.float32, device=l16.y_slots.device)
    rows16 = placed_slots(l16)
    yk[rows16] = l16.y_slots[rows16].float()
    y = yk.cpu().numpy().astype(np.float64).reshape(T, K, -1)
    ref = np.einsum("tk,tkh->th", w * keep, y)
    err = np.abs(out32.cpu().numpy() - ref).max() / max(np.abs(ref).max(), 1e-30)
    say(f"{label}: bf16 slot rows exact, combine rel err {err:.2e} against float64")
    assert err <= 1e-6, (label, err)


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8", "prefill_fp4"])
@pytest.mark.parametrize("B", [16, 64, 128])
def test_bf16_slot_rows_small_all_tokens(name, B):
    dev = device()
    over = dict(T=300, H=512, I=256, E=12)
    if name == "decode_bf16":
        over.update(K=4, n_group=4, topk_group=2, E=16)
    cfg = ms.scaled(name, **over)
    L = ms.make_layer(cfg, device=dev)
    l32, _ = forward(cfg, L, B, torch.float32)
    l16, out16 = forward(cfg, L, B, torch.bfloat16)
    label = f"{name} small B={B}"
    check_rounding_and_combine(l32, l16, label)
    ids, w, toks, ref, yref = oracle_layer_cached(f"bf16-slots-{name}-small", cfg, L)
    compare_out(out16, toks, ref, cfg["dtype"], label + " bf16 slots")
    compare_slots(l16.y_slots, toks, ids, yref, cfg["dtype"], label + " bf16 slots")


def test_bf16_slot_rows_one_stage_schedule():
    # the persistent one-launch schedule writes the same bf16 rows
    dev = device()
    for name in ("prefill_fp8", "prefill_fp4"):
        cfg = ms.scaled(name, T=400, H=512, I=256, E=8)
        L = ms.make_layer(cfg, device=dev)
        a, out_a = forward(cfg, L, 64, torch.bfloat16)
        b, out_b = forward(cfg, L, 64, torch.bfloat16, schedule="fused")
        rows = placed_slots(a)
        assert torch.equal(a.y_slots[rows].view(torch.int16), b.y_slots[rows].view(torch.int16)), name
        assert torch.equal(out_a, out_b), name
        assert b.fused_status() == 0


def test_bf16_slot_rows_prefill_fp8_full_size():
    dev = device()
    cfg = ms.CONFIGS["prefill_fp8"]
    say("generating prefill fp8 weights (32 + 1 shared experts, 1.45 GB)")
    L = ms.make_layer(cfg, device=dev)
    l32, _ = forward(cfg, L, 128, torch.float32)
    l16, out16 = forward(cfg, L, 128, torch.bfloat16)
    check_rounding_and_combine(l32, l16, "prefill fp8 B=128")
    del l32
    ids, w, toks, ref, yref = oracle_layer_cached("prefill_fp8", cfg, L)
    compare_out(out16, toks, ref, cfg["dtype"], "prefill fp8 B=128 bf16 slots")
    compare_slots(l16.y_slots, toks, ids, yref, cfg["dtype"], "prefill fp8 B=128 bf16 slots")
    del L, l16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["prefill_bf16_512", "prefill_fp8_512"])
def test_bf16_slot_rows_512_per_expert(name):
    dev = device()
    cfg = ms.CONFIGS[name]
    say(f"generating {name} weights")
    L = ms.make_layer(cfg, device=dev)
    l32, _ = forward(cfg, L, 128, torch.float32)
    l16, out16 = forward(cfg, L, 128, torch.bfloat16)
    check_rounding_and_combine(l32, l16, f"{name} B=128")
    del l32
    ids, w, toks, ref, yref = oracle_layer_cached(name, cfg, L, seeded_subset(cfg["T"], 256, 5))
    compare_out(out16, toks, ref, cfg["dtype"], f"{name} B=128 bf16 slots")
    compare_slots(l16.y_slots, toks, ids, yref, cfg["dtype"], f"{name} B=128 bf16 slots")
    del L, l16
    torch.cuda.empty_cache()


def test_bf16_slot_rows_with_skipped_ids():
    # slots whose id is outside [0,E) (experts of another GPU, in an
    # expert-parallel dispatch) are neither written nor summed
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=300, H=512, I=256, E=8)
    L = ms.make_layer(cfg, device=dev)
    layers = []
    for slot_dtype in (torch.float32, torch.bfloat16):
        layer = make_gpu_layer(cfg, L, 64, top1=False, slot_dtype=slot_dtype)
        layer.route(L["logits"], L["bias"])
        ids = layer.topk_ids.cpu().numpy()
        rng = np.random.default_rng(3)
        drop = rng.random(ids.shape) < 0.4
        ids[drop] = np.where(rng.random(ids.shape) < 0.5, -1, layer.E_slabs + 3)[drop]
        layer.topk_ids.copy_(torch.from_numpy(ids))
        layer.align()
        layer.ffn(L["x"])
        layer.combine()
        torch.cuda.synchronize()
        layers.append(layer)
    check_rounding_and_combine(layers[0], layers[1], "prefill fp8 small, 40% skipped ids")
