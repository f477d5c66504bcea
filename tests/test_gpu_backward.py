"""The backward (training) on the GPU against the oracle's derivative.

dx, dW13 and dW2 within 2e-2 * max|oracle| (bf16 GEMM operands, fp32
accumulation, as the forward's bf16 bar); the combine weights' gradient
and d_logits within 1e-5 * max|oracle| (fp32 dot products).  The oracle gets
the GPU forward's routing, weights and y_slots, so both differentiate the
same forward."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe
from gpu_helpers import device, host_bits, rel_err, say

pytestmark = pytest.mark.gpu


def run(cfg, L, B, seed=3, train=False):
    dev = device()
    layer = moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"],
                         n_group=cfg["n_group"], topk_group=cfg["topk_group"], renormalize=cfg["renormalize"],
                         shared=bool(cfg.get("shared")), x_dtype=L["x"].dtype, train=train)
    layer.forward(L["x"], L["logits"], L["bias"])
    d_out = torch.tensor(np.random.default_rng(seed).standard_normal((cfg["T"], cfg["H"])).astype(np.float32),
                         device=dev)
    dx, dw13, dw2, d_logits, dwk = layer.backward(L["x"], L["logits"], d_out)
    torch.cuda.synchronize()
    return layer, d_out, dx, dw13, dw2, d_logits, dwk


def check_all(cfg, L, B, label, train=False):
    layer, d_out, dx, dw13, dw2, d_logits, dwk = run(cfg, L, B, train=train)
    ids = layer.topk_ids.cpu().numpy()
    w = layer.topk_weights.cpu().numpy()
    y = layer.y_slots.cpu().numpy()
    rdx, rdw13, rdw2, rdwk = oracle.ffn_backward(host_bits(L["x"]), host_bits(L["w13"]), host_bits(L["w2"]), ids, w,
                                                 y, d_out.cpu().numpy(), w_dtype="bf16", x_dtype="bf16",
                                                 inter="bf16")
    rdl = oracle.route_backward(L["logits"].cpu().numpy(), ids, dwk.cpu().numpy(), cfg["K"], score=cfg["score"],
                                renormalize=cfg["renormalize"], append_shared=bool(cfg.get("shared")))
    errs = {"dx": rel_err(dx.cpu().numpy(), rdx), "dw13": rel_err(dw13.cpu().numpy(), rdw13),
            "dw2": rel_err(dw2.cpu().numpy(), rdw2), "d_w": rel_err(dwk.cpu().numpy(), rdwk),
            "d_logits": rel_err(d_logits.cpu().numpy(), rdl)}
    say(f"{label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k in ("dx", "dw13", "dw2"):
        assert errs[k] <= 2e-2, (k, errs[k])
    assert errs["d_w"] <= 1e-5 and errs["d_logits"] <= 1e-5, errs


@pytest.mark.parametrize("train", [False, True])
@pytest.mark.parametrize("B", [64, 128, 256])
def test_backward_small_softmax(B, train):
    dev = device()
    cfg = ms.scaled("tiny_fp32", T=160, H=512, I=256, E=6, K=2, dtype="bf16", B=B)
    L = ms.make_layer(cfg, device=dev)
    check_all(cfg, L, B, f"backward softmax top-2 B={B}" + (" (gate/up kept by the forward)" if train else ""),
              train=train)


@pytest.mark.parametrize("B", [64, 128])
def test_training_forward_keeps_gate_up(B):
    # the training forward: same output and slot rows as the plain forward, the
    # kept gate/up values equal x . w13[e] of every placed row, and the
    # backward that reads them agrees with the one that recomputes them
    dev = device()
    cfg = ms.scaled("tiny_fp32", T=160, H=512, I=256, E=6, K=2, dtype="bf16", B=B)
    L = ms.make_layer(cfg, device=dev)
    mk = lambda train: moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"],
                                    renormalize=cfg["renormalize"], x_dtype=L["x"].dtype, train=train,
                                    top1=False)
    a, b = mk(True), mk(False)
    oa = a.forward(L["x"], L["logits"]).clone()
    ob = b.forward(L["x"], L["logits"])
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(a.y_slots, b.y_slots)
    K, T, I = cfg["K"], cfg["T"], cfg["I"]
    P = int(a.ntpp.item())
    srt = a.sorted.cpu().numpy()[:P]
    rows = np.nonzero(srt < T * K)[0]
    toks = srt[rows] // K
    exps = a.expert_ids.cpu().numpy()[rows // B]
    xh = L["x"].double().cpu().numpy()
    wh = L["w13"].double().cpu().numpy()
    ref = np.einsum("rh,rjh->rj", xh[toks], wh[exps])              # [rows, 2I] in float64
    got = a.gate_up.cpu().numpy()[rows]
    err = rel_err(got, ref)
    assert err <= 1e-5, err
    d_out = torch.tensor(np.random.default_rng(5).standard_normal((T, cfg["H"])).astype(np.float32), device=dev)
    ga = a.backward(L["x"], L["logits"], d_out)
    gb = b.backward(L["x"], L["logits"], d_out)
    torch.cuda.synchronize()
    names = ("dx", "dw13", "dw2", "d_logits", "d_w")
    diffs = {n: rel_err(u.cpu().numpy(), v.cpu().numpy()) for n, u, v in zip(names, ga, gb)}
    say(f"B={B}: kept gate/up within {err:.1e} of x.w13; kept vs recomputed: "
        + "  ".join(f"{k} {v:.1e}" for k, v in diffs.items()))
    assert torch.equal(ga[3], gb[3]) and torch.equal(ga[4], gb[4])      # from y_slots only
    for n in ("dx", "dw13", "dw2"):
        assert diffs[n] <= 5e-3, (n, diffs[n])


def test_backward_small_sigmoid_groups_shared():
    dev = device()
    cfg = ms.scaled("decode_bf16", T=120, H=512, I=256, E=16, K=4, n_group=4, topk_group=2, shared=True)
    L = ms.make_layer(cfg, device=dev)
    check_all(cfg, L, 64, "backward sigmoid groups + shared B=64")


def test_backward_skipped_slots_and_empty_experts():
    dev = device()
    rng = np.random.default_rng(9)
    T, K, E, H, I, B = 70, 3, 9, 256, 256, 64
    cfg = ms.scaled("tiny_fp32", T=T, H=H, I=I, E=E, K=K, dtype="bf16", B=B)
    L = ms.make_layer(cfg, device=dev)
    ids = rng.integers(0, 5, (T, K)).astype(np.int32)       # experts 5..8 get no rows
    ids[rng.random((T, K)) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    tid, tw = torch.tensor(ids, device=dev), torch.tensor(w, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    y = moe.moe_grouped_ffn(L["x"], L["w13"], L["w2"], al["sorted_token_ids"], al["expert_ids"],
                            al["num_tokens_post_padded"], K=K, B=B)
    d_out = torch.tensor(rng.standard_normal((T, H)).astype(np.float32), device=dev)
    dx, dw13, dw2, dwk = moe.moe_ffn_backward(L["x"], L["w13"], L["w2"], tid, tw, al["sorted_token_ids"],
                                              al["expert_ids"], al["num_tokens_post_padded"],
                                              al["expert_offsets"], y, d_out, B=B)
    torch.cuda.synchronize()
    rdx, rdw13, rdw2, rdwk = oracle.ffn_backward(host_bits(L["x"]), host_bits(L["w13"]), host_bits(L["w2"]), ids, w,
                                                 y.cpu().numpy(), d_out.cpu().numpy(), w_dtype="bf16",
                                                 x_dtype="bf16", inter="bf16")
    assert rel_err(dx.cpu().numpy(), rdx) <= 2e-2
    assert rel_err(dw13.cpu().numpy(), rdw13) <= 2e-2
    assert rel_err(dw2.cpu().numpy(), rdw2) <= 2e-2
    assert rel_err(dwk.cpu().numpy(), rdwk) <= 1e-5
    assert not dw13[5:].any() and not dw2[5:].any()          # experts with no rows: zero
    assert (dwk.cpu().numpy()[ids < 0] == 0).all()


def test_backward_full_size_prefill_sampled():
    dev = device()
    cfg = ms.CONFIGS["prefill_bf16"]
    L = ms.make_layer(cfg, device=dev)
    layer, d_out, dx, dw13, dw2, d_logits, dwk = run(cfg, L, 64)
    ids = layer.topk_ids.cpu().numpy()
    w = layer.topk_weights.cpu().numpy()
    y = layer.y_slots.cpu().numpy()
    e = int(ids[0, 0])
    toks = np.nonzero(ids[:, 0] == e)[0]                    # every token of one expert (64)
    sub_ids = np.zeros((len(toks), 1), np.int32)
    sel = torch.tensor([e], device=dev)
    rdx, rdw13, rdw2, rdwk = oracle.ffn_backward(
        host_bits(L["x"][torch.as_tensor(toks, device=dev)]), host_bits(L["w13"].index_select(0, sel)),
        host_bits(L["w2"].index_select(0, sel)), sub_ids, w[toks], y[toks], d_out.cpu().numpy()[toks],
        w_dtype="bf16", x_dtype="bf16", inter="bf16")
    errs = (rel_err(dx.cpu().numpy()[toks], rdx), rel_err(dw13[e].cpu().numpy(), rdw13[0]),
            rel_err(dw2[e].cpu().numpy(), rdw2[0]), rel_err(dwk.cpu().numpy()[toks], rdwk))
    say(f"prefill bf16 full size, expert {e} ({len(toks)} tokens): dx {errs[0]:.2e} dw13 {errs[1]:.2e} "
        f"dw2 {errs[2]:.2e} d_w {errs[3]:.2e}")
    assert max(errs[:3]) <= 2e-2 and errs[3] <= 1e-5
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [64, 128])
def test_bf16_weight_gradients(B):
    # bf16 weight gradients are the fp32 sums rounded once (torch's RNE cast of
    # the fp32 gradients, bit for bit); every other output is unchanged
    dev = device()
    cfg = ms.scaled("tiny_fp32", T=160, H=512, I=256, E=6, K=2, dtype="bf16", B=B)
    L = ms.make_layer(cfg, device=dev)
    d_out = torch.tensor(np.random.default_rng(7).standard_normal((cfg["T"], cfg["H"])).astype(np.float32),
                         device=dev)
    res = []
    for gd in (torch.float32, torch.bfloat16):
        layer = moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"],
                             renormalize=cfg["renormalize"], x_dtype=L["x"].dtype, train=True, grad_dtype=gd)
        layer.forward(L["x"], L["logits"])
        res.append([t.clone() for t in layer.backward(L["x"], L["logits"], d_out)])
        torch.cuda.synchronize()
    (dx, dw13, dw2, dl, dwk), (dx_b, dw13_b, dw2_b, dl_b, dwk_b) = res
    assert dw13_b.dtype == torch.bfloat16 and dw2_b.dtype == torch.bfloat16
    assert torch.equal(dw13_b, dw13.to(torch.bfloat16)) and torch.equal(dw2_b, dw2.to(torch.bfloat16))
    assert torch.equal(dx, dx_b) and torch.equal(dl, dl_b) and torch.equal(dwk, dwk_b)
    say(f"B={B}: bf16 weight gradients equal the rounded fp32 ones; dx, d_w, d_logits unchanged")


def test_weight_gradients_many_tiles_per_workgroup():
    # dW13 has 16 x 8 x 12 = 1536 tiles and dW2 768: more than the persistent
    # weight-gradient kernel's grid at two workgroups per CU, so each workgroup
    # walks several tiles, across experts with no rows (zero K-steps) and one
    # with 256 rows (four K-steps); fp32 against the oracle, bf16 the same sums
    dev = device()
    rng = np.random.default_rng(21)
    T, K, E, H, I, B = 384, 2, 16, 1536, 512, 64
    cfg = ms.scaled("tiny_fp32", T=T, H=H, I=I, E=E, K=K, dtype="bf16", B=B)
    L = ms.make_layer(cfg, device=dev)
    ids = rng.integers(1, 12, (T, K)).astype(np.int32)      # experts 12..15 get no rows
    ids[:256, 0] = 0                                        # expert 0: 256 rows
    ids[:256, 1] = rng.integers(1, 12, 256)
    w = rng.random((T, K)).astype(np.float32)
    tid, tw = torch.tensor(ids, device=dev), torch.tensor(w, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    y = moe.moe_grouped_ffn(L["x"], L["w13"], L["w2"], al["sorted_token_ids"], al["expert_ids"],
                            al["num_tokens_post_padded"], K=K, B=B)
    d_out = torch.tensor(rng.standard_normal((T, H)).astype(np.float32), device=dev)
    res = []
    for gd in (torch.float32, torch.bfloat16):
        res.append(moe.moe_ffn_backward(L["x"], L["w13"], L["w2"], tid, tw, al["sorted_token_ids"],
                                        al["expert_ids"], al["num_tokens_post_padded"], al["expert_offsets"], y,
                                        d_out, B=B, grad_dtype=gd))
        torch.cuda.synchronize()
    (dx, dw13, dw2, dwk), (dx_b, dw13_b, dw2_b, dwk_b) = res
    rdx, rdw13, rdw2, rdwk = oracle.ffn_backward(host_bits(L["x"]), host_bits(L["w13"]), host_bits(L["w2"]), ids, w,
                                                 y.cpu().numpy(), d_out.cpu().numpy(), w_dtype="bf16",
                                                 x_dtype="bf16", inter="bf16")
    errs = (rel_err(dw13.cpu().numpy(), rdw13), rel_err(dw2.cpu().numpy(), rdw2), rel_err(dx.cpu().numpy(), rdx))
    say(f"{E} experts, H {H}, I {I}: dw13 {errs[0]:.2e} dw2 {errs[1]:.2e} dx {errs[2]:.2e}")
    assert max(errs) <= 2e-2 and rel_err(dwk.cpu().numpy(), rdwk) <= 1e-5
    assert not dw13[12:].any() and not dw2[12:].any()
    assert torch.equal(dw13_b, dw13.to(torch.bfloat16)) and torch.equal(dw2_b, dw2.to(torch.bfloat16))
    assert torch.equal(dx, dx_b) and torch.equal(dwk, dwk_b)


def test_bf16_weight_gradients_full_size():
    # at the full prefill bf16 shape the bf16 weight gradients come from the
    # persistent kernel (57344 dW13 tiles, over a hundred per workgroup) and
    # the fp32 ones from the one-tile-per-workgroup kernel: the first must be
    # the second rounded to bf16, bit for bit
    dev = device()
    cfg = ms.CONFIGS["prefill_bf16"]
    L = ms.make_layer(cfg, device=dev)
    d_out = torch.tensor(np.random.default_rng(5).standard_normal((cfg["T"], cfg["H"])).astype(np.float32),
                         device=dev)
    res = []
    for gd in (torch.float32, torch.bfloat16):
        layer = moe.MoELayer(L["w13"], L["w2"], T=cfg["T"], K=1, B=cfg["B"], score="softmax", renormalize=False,
                             train=True, grad_dtype=gd)
        layer.forward(L["x"], L["logits"])
        _, dw13, dw2, _, _ = layer.backward(L["x"], L["logits"], d_out)
        torch.cuda.synchronize()
        res.append((dw13, dw2, layer))
    (dw13, dw2, _), (dw13_b, dw2_b, _) = res
    assert torch.equal(dw13_b, dw13.to(torch.bfloat16)) and torch.equal(dw2_b, dw2.to(torch.bfloat16))
    assert dw13.abs().amax().item() > 0
    say("prefill bf16 full size: bf16 weight gradients (persistent kernel) equal the rounded fp32 ones")
    del res, L
    torch.cuda.empty_cache()
