"""Permute / unpermute and the FFN in the sorted row order on the GPU.

The permuted rows, the inverse row map and the per-row scales are compared bit
for bit with the oracle.  The layer run through permute -> FFN on sorted rows
-> unpermute-combine must give the same bits as the layer that gathers rows
inside the FFN (the GEMMs see the same operands in the same order and the two
combines share their arithmetic), and both are within tolerance of the
oracle."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe
from gpu_helpers import (TOL, compare_out, compare_slots, device, make_gpu_layer, oracle_layer_cached,
                         oracle_tokens, rel_err, route_oracle, say)

pytestmark = pytest.mark.gpu


def ids_with_invalid(rng, T, K, E, p_bad=0.05):
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    bad = rng.random((T, K)) < p_bad
    ids[bad] = rng.choice([-1, E, E + 7], size=int(bad.sum()))
    return ids


@pytest.mark.parametrize("T,K,E,B,width,dt", [
    (1, 1, 1, 16, 16, torch.uint8), (37, 3, 5, 16, 48, torch.uint8), (300, 8, 64, 32, 512, torch.bfloat16),
    (2048, 1, 32, 64, 7168, torch.bfloat16), (16384, 8, 256, 64, 64, torch.float32),
    (999, 2, 33, 128, 7168, torch.uint8)])
def test_permute_rows_match_oracle(T, K, E, B, width, dt):
    dev = device()
    rng = np.random.default_rng(T + width)
    ids = ids_with_invalid(rng, T, K, E)
    tid = torch.tensor(ids, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    if dt == torch.float32:
        x = torch.tensor(rng.standard_normal((T, width)).astype(np.float32), device=dev)
    else:
        x = torch.tensor(rng.integers(0, 255, (T, width * (2 if dt == torch.bfloat16 else 1))).astype(np.uint8),
                         device=dev).view(dt)
    scale = torch.tensor(rng.random(T).astype(np.float32) + 0.5, device=dev)
    C = al["sorted_token_ids"].numel()
    # rows past the padded count must keep what was there
    xp0 = torch.full((C, x[0].numel() * x.element_size()), 7, dtype=torch.uint8, device=dev)
    xp0 = xp0.view(dt).view((C,) + tuple(x.shape[1:]))
    sp0 = torch.full((C,), -3.0, dtype=torch.float32, device=dev)
    xp, ros, sp = moe.moe_permute_rows(x, tid, al["sorted_token_ids"], al["num_tokens_post_padded"], E, B,
                                       x_scale=scale, x_perm=xp0.clone(), x_perm_scale=sp0.clone())
    torch.cuda.synchronize()
    srt = al["sorted_token_ids"].cpu().numpy()
    P = int(al["num_tokens_post_padded"].item())
    u8 = lambda t: t.cpu().contiguous().view(torch.uint8).numpy()
    want = oracle.permute_rows(u8(x), srt, K, P=P, out=u8(xp0))
    assert np.array_equal(u8(xp), want)
    assert np.array_equal(ros.cpu().numpy(), oracle.row_of_slot(srt, T * K))
    assert np.array_equal(sp.cpu().numpy(),
                          oracle.permute_rows(scale.cpu().numpy(), srt, K, P=P, out=sp0.cpu().numpy()))
    say(f"permute T={T} K={K} E={E} B={B} row {u8(x).shape[1]} B, P={P} of C={C}: bit-exact")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_unpermute_combine_equals_combine(out_dtype):
    dev = device()
    rng = np.random.default_rng(5)
    T, K, E, B, H = 513, 6, 40, 32, 1024
    ids = ids_with_invalid(rng, T, K, E)
    tid = torch.tensor(ids, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    y_slots = torch.tensor(rng.standard_normal((T * K, H)).astype(np.float32), device=dev)
    w = torch.tensor(rng.random((T, K)).astype(np.float32), device=dev)
    # slot rows moved into the sorted order (row r holds slot sorted[r])
    srt = al["sorted_token_ids"]
    C = srt.numel()
    placed = srt < T * K
    y_perm = torch.zeros((C, H), dtype=torch.float32, device=dev)
    y_perm[placed] = y_slots[srt[placed].long()]
    _, ros, _ = moe.moe_permute_rows(torch.zeros((T, 16), dtype=torch.uint8, device=dev), tid, srt,
                                     al["num_tokens_post_padded"], E, B)
    a = moe.moe_unpermute_combine(y_perm, w, ros, out_dtype=out_dtype)
    b = moe.moe_combine(y_slots, w, tid, E, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.unpermute_combine(y_perm.cpu().numpy(), w.cpu().numpy(), ros.cpu().numpy())
    assert rel_err(a.float().cpu().numpy(), ref) <= (1e-6 if out_dtype == torch.float32 else 8e-3)


def sorted_vs_gather(cfg, L, B):
    dev = device()
    g = make_gpu_layer(cfg, L, B, top1=False)                 # its slot rows are compared
    out_g = g.forward(L["x"], L["logits"], L["bias"]).clone()
    yg = g.y_slots.clone()
    w13, w2, s13, s2 = L["w13"], L["w2"], L.get("w13_scale"), L.get("w2_scale")
    if cfg["dtype"] == "e2m1":
        w13, w2, s13, s2 = w13.view(moe.FP4), w2.view(moe.FP4), s13.view(moe.E8M0), s2.view(moe.E8M0)
    s = moe.MoELayer(w13, w2, T=cfg["T"], K=cfg["K"], B=B, score=cfg["score"], n_group=cfg["n_group"],
                     topk_group=cfg["topk_group"], renormalize=cfg["renormalize"],
                     shared=bool(cfg.get("shared")), w13_scale=s13, w2_scale=s2, x_dtype=L["x"].dtype,
                     out_dtype=torch.bfloat16, rows="sorted")
    out_s = s.forward(L["x"], L["logits"], L["bias"])
    torch.cuda.synchronize()
    srt = s.sorted
    placed = srt < s.T * s.KO
    assert torch.equal(s.sorted, g.sorted)
    assert torch.equal(s.y_slots[placed], yg[srt[placed].long()])       # same rows, same bits
    assert torch.equal(out_s, out_g)
    return s, out_s


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_fp8", "prefill_fp4"])
def test_layer_sorted_rows_equal_gathered_rows(name):
    dev = device()
    if name == "decode_bf16":
        cfg = ms.scaled(name, T=150, H=512, I=256, E=16, K=4, n_group=4, topk_group=2)
    else:
        cfg = ms.scaled(name, T=201, H=768, I=384, E=12)
    L = ms.make_layer(cfg, device=dev)
    for B in (16, 64, 128):
        s, out = sorted_vs_gather(cfg, L, B)
        ids, w = route_oracle(cfg, L)
        ref, _ = oracle_tokens(L["x"], L["w13"], L["w2"], ids, w, np.arange(cfg["T"]),
                               L.get("w13_scale"), L.get("w2_scale"))
        err = rel_err(out.float().cpu().numpy(), ref)
        say(f"{name} sorted rows B={B}: bit-identical to the gathered path, rel err {err:.3e}")
        assert err <= TOL[cfg["dtype"]]


def test_layer_sorted_rows_full_size_prefill():
    dev = device()
    cfg = ms.CONFIGS["prefill_bf16"]
    L = ms.make_layer(cfg, device=dev)
    s, out = sorted_vs_gather(cfg, L, 64)
    say("prefill bf16 full size: sorted rows bit-identical to gathered rows")
    # every token against the oracle; the sorted rows read back by slot
    ids, w, toks, ref, yref = oracle_layer_cached("prefill_bf16", cfg, L)
    compare_out(out, toks, ref, cfg["dtype"], "prefill bf16 sorted rows, B 64")
    ros = s.row_of_slot.long()
    y_by_slot = torch.zeros((s.T * s.KO, s.H), dtype=torch.float32, device=dev)
    y_by_slot[ros >= 0] = s.y_slots[ros[ros >= 0]]
    compare_slots(y_by_slot, toks, ids, yref, cfg["dtype"], "prefill bf16 sorted rows, B 64")
    del L
    torch.cuda.empty_cache()


# ----------------------------------------------- gradient of the unpermute --
@pytest.mark.parametrize("T,K,E,B,H,dt", [
    (1, 1, 1, 16, 4, torch.float32), (37, 3, 5, 16, 48, torch.float32), (300, 8, 64, 32, 512, torch.bfloat16),
    (2048, 1, 32, 64, 7168, torch.float32), (16384, 8, 256, 64, 64, torch.bfloat16),
    (999, 2, 33, 128, 7168, torch.bfloat16)])
def test_unpermute_combine_backward_matches_oracle(T, K, E, B, H, dt):
    dev = device()
    say(f"unpermute backward T={T} K={K} E={E} B={B} H={H} {dt}")
    rng = np.random.default_rng(T * 7 + H)
    ids = ids_with_invalid(rng, T, K, E)
    tid = torch.tensor(ids, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    srt_d, ntpp = al["sorted_token_ids"], al["num_tokens_post_padded"]
    C = srt_d.numel()
    g = rng.standard_normal((T, H)).astype(np.float32)
    y = rng.standard_normal((C, H)).astype(np.float32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    # rows past the padded count keep what was there; every weight gradient is written
    dy0 = torch.full((C, H), 7.0, dtype=dt, device=dev)
    dw0 = torch.full((T, K), -999.0, dtype=torch.float32, device=dev)
    dy, dw = moe.moe_unpermute_combine_backward(
        torch.tensor(g, device=dev), torch.tensor(y, device=dev), torch.tensor(w, device=dev), tid, srt_d, ntpp,
        E, B, d_y_perm_dtype=dt, d_y_perm=dy0.clone(), d_topk_weights=dw0.clone())
    torch.cuda.synchronize()
    srt = srt_d.cpu().numpy()
    P = int(ntpp.item())
    want_dy, want_dw = oracle.unpermute_combine_backward(g, y, w, srt, P=P,
                                                         round_to="f32" if dt == torch.float32 else "bf16")
    got_dy = dy.float().cpu().numpy()
    assert np.array_equal(got_dy[:P], want_dy.astype(np.float32))                # one product, one rounding
    assert (got_dy[P:] == 7.0).all()
    got_dw = dw.cpu().numpy()
    assert not (got_dw == -999.0).any()
    ros = oracle.row_of_slot(srt, T * K)
    skipped = (ros < 0).reshape(T, K)
    assert (got_dw[skipped] == 0).all()
    # fp32 sums in another order: within 1e-5 of each slot's sum of |terms|
    scale = np.zeros((T, K))
    placed = np.nonzero(ros >= 0)[0]
    scale.ravel()[placed] = np.abs(g[placed // K].astype(np.float64) * y[ros[placed]]).sum(axis=1)
    err = np.abs(got_dw - want_dw)
    assert (err <= 1e-5 * scale + 1e-30).all(), float((err / np.maximum(scale, 1e-30)).max())
    say(f"  P={P} of C={C}: d_y_perm bit-exact, d_w within {float((err / np.maximum(scale, 1e-30)).max()):.1e}")


@pytest.mark.parametrize("T,K,E,B,H", [(37, 3, 5, 16, 48), (2048, 8, 32, 64, 512)])
def test_unit_weight_unpermute_is_the_permute_gradient(T, K, E, B, H):
    # d_x[t] = sum of the rows of t's slots: the unweighted unpermute, which
    # must also give the same bits as the weighted call with weights of 1
    dev = device()
    rng = np.random.default_rng(T + 3)
    ids = ids_with_invalid(rng, T, K, E)
    tid = torch.tensor(ids, device=dev)
    al = moe.moe_align_sort(tid, E, B)
    C = al["sorted_token_ids"].numel()
    _, ros, _ = moe.moe_permute_rows(torch.zeros((T, 16), dtype=torch.uint8, device=dev), tid,
                                     al["sorted_token_ids"], al["num_tokens_post_padded"], E, B)
    d_xp = rng.standard_normal((C, H)).astype(np.float32)
    d_xp_d = torch.tensor(d_xp, device=dev)
    dx = moe.moe_unpermute_combine(d_xp_d, None, ros, out_dtype=torch.float32, T=T, K=K)
    ones = torch.ones((T, K), dtype=torch.float32, device=dev)
    dx1 = moe.moe_unpermute_combine(d_xp_d, ones, ros, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx1)
    want = oracle.unpermute_combine(d_xp, np.ones((T, K), np.float32), ros.cpu().numpy())
    scale = oracle.unpermute_combine(np.abs(d_xp), np.ones((T, K), np.float32), ros.cpu().numpy())
    assert (np.abs(dx.cpu().numpy() - want) <= 1e-6 * scale + 1e-30).all()
    say(f"unit-weight unpermute T={T} K={K}: equals the weighted call, within 1e-6 of the oracle")
