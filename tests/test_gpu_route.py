"""Top-k routing on the GPU against the oracle: ids exact, weights within 1e-6
relative (both sides form the scores in double and decide on fp32 keys)."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe
from gpu_helpers import device, say

pytestmark = pytest.mark.gpu


def compare(logits_np, K, bias_np=None, **kw):
    dev = device()
    logits = torch.from_numpy(np.ascontiguousarray(logits_np, np.float32)).to(dev)
    bias = None if bias_np is None else torch.from_numpy(np.asarray(bias_np, np.float32)).to(dev)
    ids, w = moe.moe_route_topk(logits, K, bias=bias, **kw)
    torch.cuda.synchronize()
    rid, rw = oracle.route_topk(logits_np, K, bias=bias_np, **kw)
    gid = ids.cpu().numpy()
    gw = w.cpu().numpy()
    bad = np.flatnonzero(np.any(gid != rid, axis=1))
    assert bad.size == 0, f"{bad.size} tokens differ, e.g. t={bad[0]}: {gid[bad[0]]} vs {rid[bad[0]]}"
    assert np.allclose(gw, rw, rtol=1e-6, atol=0), np.abs(gw - rw).max()
    return gid, gw


def test_route_tiny_softmax_top2():
    cfg = ms.CONFIGS["tiny_fp32"]
    L = ms.make_layer(cfg, weights=False)
    say("route tiny softmax top-2 of 8")
    compare(L["logits"].numpy(), 2, score="softmax", renormalize=True)


def test_route_decode_sigmoid_bias_groups():
    cfg = ms.CONFIGS["decode_bf16"]
    L = ms.make_layer(cfg, weights=False)
    say("route decode sigmoid+bias, 8 groups keep 4, top-8 of 256")
    compare(L["logits"].numpy(), 8, L["bias"].numpy(), score="sigmoid", n_group=8, topk_group=4,
            renormalize=True)


def test_route_prefill_assignments_and_shared():
    for name in ("prefill_bf16", "prefill_fp8"):
        cfg = ms.CONFIGS[name]
        L = ms.make_layer(cfg, weights=False)
        say(f"route {name}")
        gid, gw = compare(L["logits"].numpy(), 1, score="softmax", renormalize=False,
                          append_shared=bool(cfg.get("shared")))
        assert np.array_equal(gid[:, 0], ms.assigned_experts(cfg))
        if cfg.get("shared"):
            assert np.all(gid[:, 1] == cfg["E"]) and np.all(gw[:, 1] == 1.0)


@pytest.mark.parametrize("E,K,n_group,topk_group,score", [
    (8, 1, 1, 1, "softmax"), (16, 4, 4, 2, "sigmoid"), (64, 6, 1, 1, "sigmoid"),
    (256, 8, 8, 4, "sigmoid"), (256, 8, 1, 1, "softmax"), (1024, 16, 16, 3, "sigmoid"),
    (160, 6, 1, 1, "softmax"), (64, 64, 1, 1, "softmax"), (96, 5, 32, 4, "sigmoid"),
    # group sizes on both paths of the group scores: 128 lanes (two registers,
    # a scan), 2 lanes with E not a multiple of 64, 1 expert per group
    (1024, 8, 8, 2, "sigmoid"), (40, 3, 20, 5, "sigmoid"), (8, 2, 8, 3, "sigmoid")])
def test_route_random(E, K, n_group, topk_group, score):
    rng = np.random.default_rng(E * 100 + K)
    T = 517
    logits = rng.normal(0, 2, size=(T, E)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, size=E).astype(np.float32) if score == "sigmoid" else None
    say(f"route random E={E} K={K} groups={n_group}/{topk_group} {score}")
    compare(logits, K, bias, score=score, n_group=n_group, topk_group=topk_group, renormalize=True,
            routed_scaling=2.5)
    compare(logits, K, bias, score=score, n_group=n_group, topk_group=topk_group, renormalize=False,
            append_shared=True)


def test_route_ties_choose_lower_ids():
    logits = np.zeros((9, 32), np.float32)
    logits[3, 20] = 1.0
    logits[4, 5:9] = 0.5
    gid, _ = compare(logits, 4, score="softmax")
    assert gid[0].tolist() == [0, 1, 2, 3] and gid[3].tolist() == [20, 0, 1, 2]
    assert gid[4].tolist() == [5, 6, 7, 8]


@pytest.mark.parametrize("gsize", [4, 32, 24])
def test_route_group_score_ties_choose_lower_groups(gsize):
    # every group scores the same, so the kept groups are the lowest indices;
    # inside them the keys decide (gsize 24 takes the scanning path)
    n_group = 8
    E = gsize * n_group
    T = 64
    rng = np.random.default_rng(gsize)
    logits = np.zeros((T, E), np.float32)
    for t in range(T):
        for g in range(n_group):
            # the same two largest keys in every group, different smaller ones
            base = g * gsize
            logits[t, base + rng.integers(gsize)] = 3.0
            rest = [i for i in range(base, base + gsize) if logits[t, i] == 0.0]
            logits[t, rest[rng.integers(len(rest))]] = 2.0
    gid, _ = compare(logits, 4, None, score="sigmoid", n_group=n_group, topk_group=3, renormalize=True)
    assert (gid // gsize < 3).all(), "groups 0..2 must be kept on equal scores"
