"""The grouped FFN and the whole layer (route -> align -> FFN -> combine) on the
GPU against the oracle: max|gpu - oracle| <= tol * max|oracle| with tol 1e-4
(fp32), 2e-2 (bf16), 6e-2 (fp8 and MXFP4 weights, both with fp8 activations),
over the layer output and, with the same bar, over the slot rows y_slots.
Every token is compared, at the small shapes and at the full decode and
prefill shapes; the compute-bound shapes with 512 tokens per expert (top-8 of
32 experts) are compared on a seeded subset of 256 tokens."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe
from gpu_helpers import (TOL, compare_out, compare_slots, device, make_gpu_layer, oracle_layer_cached,
                         oracle_tokens, rel_err, route_oracle, say, seeded_subset, host_bits)

pytestmark = pytest.mark.gpu


def run_layer(cfg, L, B=None):
    """The layer's forward as a caller runs it.  A top-1 layer runs the FFN and
    the combine as one call (no slot rows written); it is also run through the
    separate FFN + combine, which must give the same output bits, so that its
    slot rows are there to compare as well."""
    layer = make_gpu_layer(cfg, L, B)
    out = layer.forward(L["x"], L["logits"], L["bias"]).clone()
    if layer.top1:
        layer.ffn(L["x"])
        sep = layer.combine()
        torch.cuda.synchronize()
        assert torch.equal(sep, out), "top-1 FFN + combine differs from the separate calls"
    torch.cuda.synchronize()
    return layer, out


def check_routing_and_align(cfg, L, layer, ids, w, label):
    gid = layer.topk_ids.cpu().numpy()
    assert np.array_equal(gid, ids), f"{label}: routing differs"
    assert np.allclose(layer.topk_weights.cpu().numpy(), w, rtol=1e-6, atol=0)
    al = oracle.align_sort(ids, layer.E_slabs, layer.B)
    assert np.array_equal(layer.sorted.cpu().numpy(), al["sorted_token_ids"]), f"{label}: align"
    assert np.array_equal(layer.expert_ids.cpu().numpy(), al["expert_ids"]), f"{label}: expert_ids"
    assert int(layer.ntpp.item()) == al["num_tokens_post_padded"]


def check_layer(cfg, L, toks=None, B=None, label="", name=None):
    """Routing and Align & Sort bit-exact, then the output rows of ``toks``
    (every token when None) and their slot rows within the dtype's tolerance.
    ``name`` caches the oracle's result under that workload name, so several
    block sizes (and other test files) share one oracle run."""
    layer, out = run_layer(cfg, L, B)
    if name is not None:
        ids, w, toks, ref, yref = oracle_layer_cached(name, cfg, L, toks)
    else:
        ids, w = route_oracle(cfg, L)
        toks = np.arange(cfg["T"]) if toks is None else np.asarray(toks)
        ref, yref = oracle_tokens(L["x"], L["w13"], L["w2"], ids, w, toks, L.get("w13_scale"),
                                  L.get("w2_scale"))
    check_routing_and_align(cfg, L, layer, ids, w, label)
    compare_out(out, toks, ref, cfg["dtype"], label)
    compare_slots(layer.y_slots, toks, ids, yref, cfg["dtype"], label)
    return layer, out


def test_layer_tiny_fp32():
    dev = device()
    cfg = ms.CONFIGS["tiny_fp32"]
    L = ms.make_layer(cfg, device=dev)
    check_layer(cfg, L, np.arange(cfg["T"]), label="tiny fp32 B=16")


@pytest.mark.parametrize("B", [16, 32, 64, 128, 256])
def test_layer_small_bf16_all_tokens(B):
    dev = device()
    cfg = ms.scaled("decode_bf16", T=300, H=512, I=384, E=16, K=4, n_group=4, topk_group=2)
    L = ms.make_layer(cfg, device=dev)
    check_layer(cfg, L, np.arange(cfg["T"]), B=B, label=f"small bf16 B={B}")


@pytest.mark.parametrize("B", [16, 32, 64, 128, 256])
def test_layer_small_fp8_all_tokens(B):
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=333, H=768, I=256, E=12)
    L = ms.make_layer(cfg, device=dev)
    check_layer(cfg, L, np.arange(cfg["T"]), B=B, label=f"small fp8 B={B}")


@pytest.mark.parametrize("B", [16, 32, 64, 128, 256])
def test_layer_small_mxfp4_all_tokens(B):
    dev = device()
    cfg = ms.scaled("prefill_fp4", T=333, H=768, I=384, E=12)
    L = ms.make_layer(cfg, device=dev)
    check_layer(cfg, L, np.arange(cfg["T"]), B=B, label=f"small mxfp4 B={B}")


def test_layer_small_mxfp4_grouped_sigmoid():
    dev = device()
    cfg = ms.scaled("decode_fp4", T=96, H=512, I=256, E=16, K=4, n_group=4, topk_group=2)
    L = ms.make_layer(cfg, device=dev)
    for B in (16, 32):
        check_layer(cfg, L, np.arange(cfg["T"]), B=B, label=f"small mxfp4 decode B={B}")


@pytest.mark.parametrize("name", ["prefill_bf16", "prefill_fp8", "prefill_fp4"])
def test_layer_blocks_ending_in_padding(name):
    """Experts with 1, 33, 65, 97, 128 and 160 tokens: at block 128 their
    blocks hold 1, 2, 3, 4, 4 and (4, 1) subtiles of 32 rows with a slot, at
    block 64 (1, 2), ...; a block whose last subtiles are all padding is
    computed as the smaller tile of its rows.  Every token against the oracle,
    and the slot rows bit-identical to block 16's."""
    dev = device()
    counts = [1, 33, 65, 97, 128, 160]
    cfg = ms.scaled(name, T=sum(counts), H=512, I=256, E=len(counts))
    L = ms.make_layer(cfg, device=dev)
    assign = np.repeat(np.arange(len(counts)), counts)[np.random.default_rng(7).permutation(cfg["T"])]
    logits = torch.zeros(cfg["T"], cfg["E"], dtype=torch.float32)
    logits[torch.arange(cfg["T"]), torch.from_numpy(assign)] = 8.0
    L["logits"] = logits.to(dev)
    ref_layer, _ = run_layer(cfg, L, 16)
    y16 = ref_layer.y_slots.clone()
    for B in (64, 128):
        layer, _ = check_layer(cfg, L, None, B=B, label=f"{name} padded blocks B={B}")
        assert torch.equal(layer.y_slots, y16), f"{name} B={B}: slot rows differ from block 16's"


def test_ffn_output_is_block_size_invariant():
    dev = device()
    for name in ("decode_bf16", "prefill_fp8", "prefill_fp4"):
        cfg = ms.scaled(name, T=200, H=256, I=256, E=8, K=2, n_group=2, topk_group=2)
        if name != "decode_bf16":
            cfg = ms.scaled(name, T=200, H=256, I=256, E=8)
        L = ms.make_layer(cfg, device=dev)
        ys = []
        for B in (16, 32, 64, 128, 256):
            layer, _ = run_layer(cfg, L, B)
            ys.append(layer.y_slots.clone())
        for y in ys[1:]:
            assert torch.equal(y, ys[0]), name


def test_packed_weights_give_identical_results():
    dev = device()
    for name in ("decode_bf16", "prefill_fp8", "prefill_fp4"):
        over = dict(T=150, H=512, I=256, E=6)
        if name == "decode_bf16":
            over.update(K=3, n_group=2, topk_group=2)
        cfg = ms.scaled(name, **over)
        L = ms.make_layer(cfg, device=dev)
        for B in (16, 64, 128, 256):
            ys = []
            for packed in (False, True):
                layer = make_gpu_layer(cfg, L, B, packed=packed, top1=False)     # compares slot rows
                layer.forward(L["x"], L["logits"], L["bias"])
                torch.cuda.synchronize()
                ys.append(layer.y_slots.clone())
            say(f"{name} B={B}: packed == canonical")
            assert torch.equal(ys[0], ys[1]), (name, B)


def test_fp8_token_quantisation_codes_match_oracle():
    dev = device()
    cfg = ms.scaled("prefill_fp8", T=257, H=1024, I=256, E=4)
    L = ms.make_layer(cfg, device=dev)
    layer, _ = run_layer(cfg, L)
    T, H = cfg["T"], cfg["H"]
    ws = layer.ws_ffn.cpu().numpy()
    codes = ws[:T * H].reshape(T, H)                         # workspace region 0: x codes
    off = (T * H + 255) // 256 * 256
    scales = ws[off:off + 4 * T].view(np.float32)             # region 1: per-token scales
    q, s = oracle.quant_tokens_e4m3(host_bits(L["x"]))
    assert np.array_equal(scales, s)
    same = (codes == q) | (((codes & 0x7F) == 0) & ((q & 0x7F) == 0))   # +0 / -0 alike
    assert same.all(), f"{(~same).sum()} codes differ"


def test_generator_device_matches_host():
    dev = device()
    cfg = ms.scaled("prefill_fp8", H=256, I=128, E=3)
    g = ms.make_weights(cfg, device=dev)
    h = ms.make_weights(cfg, device="cpu")
    for k in ("w13", "w2"):
        assert np.array_equal(host_bits(g[k]), host_bits(h[k]))
    for k in ("w13_scale", "w2_scale"):
        assert torch.equal(g[k].cpu(), h[k])
    cfg = ms.scaled("decode_bf16", H=256, I=128, E=2)
    assert torch.equal(ms.make_layer(cfg, device=dev)["x"].cpu().view(torch.int16),
                       ms.make_layer(cfg, device="cpu")["x"].view(torch.int16))
    cfg = ms.scaled("prefill_fp4", H=256, I=128, E=3)
    g = ms.make_weights(cfg, device=dev)
    h = ms.make_weights(cfg, device="cpu")
    for k in ("w13", "w2", "w13_scale", "w2_scale"):
        assert torch.equal(g[k].cpu(), h[k]), k


# ----------------------------------------------------------- full-size shapes --
# Every token of the decode and prefill workloads against the oracle, at each
# block size the bench and the pages' tuning range use; the oracle runs once
# per workload and is shared by the block sizes.

def test_layer_decode_bf16_full_size():
    dev = device()
    cfg = ms.CONFIGS["decode_bf16"]
    say("generating DeepSeek-V3-shaped decode weights (256 experts, 22.5 GB bf16)")
    L = ms.make_layer(cfg, device=dev)
    for B in (16, 32):
        check_layer(cfg, L, B=B, label=f"decode bf16 B={B}", name="decode_bf16")
    del L
    torch.cuda.empty_cache()


def test_layer_prefill_bf16_full_size():
    dev = device()
    cfg = ms.CONFIGS["prefill_bf16"]
    say("generating prefill bf16 weights (32 experts, 2.8 GB)")
    L = ms.make_layer(cfg, device=dev)
    for B in (32, 64, 128):
        check_layer(cfg, L, B=B, label=f"prefill bf16 B={B}", name="prefill_bf16")
    del L
    torch.cuda.empty_cache()


def test_layer_prefill_fp8_full_size():
    dev = device()
    cfg = ms.CONFIGS["prefill_fp8"]
    say("generating prefill fp8 weights (32 + 1 shared experts, 1.45 GB)")
    L = ms.make_layer(cfg, device=dev)
    for B in (32, 64, 128):
        check_layer(cfg, L, B=B, label=f"prefill fp8 B={B}", name="prefill_fp8")
    del L
    torch.cuda.empty_cache()


def test_layer_decode_mxfp4_full_size():
    dev = device()
    cfg = ms.CONFIGS["decode_fp4"]
    say("generating DeepSeek-V3-shaped MXFP4 decode weights (256 experts, 5.6 GB)")
    L = ms.make_layer(cfg, device=dev)
    for B in (16, 32):
        check_layer(cfg, L, B=B, label=f"decode mxfp4 B={B}", name="decode_fp4")
    del L
    torch.cuda.empty_cache()


def test_layer_prefill_mxfp4_full_size():
    dev = device()
    cfg = ms.CONFIGS["prefill_fp4"]
    say("generating prefill MXFP4 weights (32 experts, 0.7 GB)")
    L = ms.make_layer(cfg, device=dev)
    for B in (32, 64, 128):
        check_layer(cfg, L, B=B, label=f"prefill mxfp4 B={B}", name="prefill_fp4")
    del L
    torch.cuda.empty_cache()


def test_layer_prefill_fp8_uniform_full_size():
    # the pages' aiter a8w8 shape: 32 experts x 64 tokens, fp8
    dev = device()
    cfg = ms.CONFIGS["prefill_fp8_uniform"]
    say("generating prefill fp8 weights (32 experts, 1.41 GB), uniform routing")
    L = ms.make_layer(cfg, device=dev)
    for B in (32, 64):
        check_layer(cfg, L, B=B, label=f"prefill fp8 uniform B={B}", name="prefill_fp8_uniform")
    del L
    torch.cuda.empty_cache()


SUBSET_512 = 256        # tokens of the compute-bound shapes compared with the oracle


@pytest.mark.parametrize("name", ["prefill_bf16_512", "prefill_fp8_512", "prefill_fp4_512"])
def test_layer_512_per_expert_full_size(name):
    # the compute-bound shapes at the block size the bench times them with;
    # the whole layer runs, a seeded 256-token subset is compared
    dev = device()
    cfg = ms.CONFIGS[name]
    say(f"generating {name} weights; 2048 tokens x top-{cfg['K']} over {cfg['E']} experts")
    L = ms.make_layer(cfg, device=dev)
    check_layer(cfg, L, seeded_subset(cfg["T"], SUBSET_512, 5), B=128, label=f"{name} B=128", name=name)
    del L
    torch.cuda.empty_cache()
