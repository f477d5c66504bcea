"""Align & Sort on the GPU, bit-exact against the oracle's stable counting sort
(full buffers: sorted_token_ids, expert_ids, num_tokens_post_padded, offsets)."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe
from gpu_helpers import device, say

pytestmark = pytest.mark.gpu


def run_and_compare(ids_np, E, B, label=""):
    dev = device()
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).to(dev)
    say(f"align {label}: T,K={ids_np.shape} E={E} B={B}")
    r = moe.moe_align_sort(ids, E, B)
    torch.cuda.synchronize()
    ref = oracle.align_sort(ids_np, E, B)
    assert int(r["num_tokens_post_padded"].item()) == ref["num_tokens_post_padded"], label
    assert np.array_equal(r["expert_offsets"].cpu().numpy(), ref["expert_offsets"]), label
    assert np.array_equal(r["expert_ids"].cpu().numpy(), ref["expert_ids"]), label
    got = r["sorted_token_ids"].cpu().numpy()
    want = ref["sorted_token_ids"]
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError(f"{label}: {bad.size} positions differ, first {bad[:8]} "
                             f"got {got[bad[:8]]} want {want[bad[:8]]}")
    return r


def test_align_16k_top8_of_256_block64():
    cfg = ms.CONFIGS["align_16k"]
    ids = ms.zipf_topk_ids(0, ms.TAG_IDS, cfg["T"], cfg["K"], cfg["E"], cfg["zipf_s"])
    run_and_compare(ids, cfg["E"], cfg["B"], "16384x8/256 Zipf1.1")


@pytest.mark.parametrize("T", [64, 1024, 131072, 1048576])
def test_align_size_sweep(T):
    ids = ms.zipf_topk_ids(0, ms.TAG_IDS, T, 8, 256, 1.1)
    run_and_compare(ids, 256, 64, f"sweep T={T}")


@pytest.mark.parametrize("B", [1, 16, 32, 64, 128])
def test_align_decode_and_prefill_shapes(B):
    rng = np.random.default_rng(B)
    run_and_compare(rng.integers(0, 256, size=(64, 8)).astype(np.int32), 256, B, "decode 64x8")
    run_and_compare(rng.integers(0, 33, size=(2048, 2)).astype(np.int32), 33, B, "prefill 2048x2/33")


def test_align_random_shapes_and_edges():
    rng = np.random.default_rng(7)
    cases = []
    for T in (0, 1, 2, 3, 17, 511, 512, 513, 4095, 4097, 20000):
        for K in (1, 2, 8):
            E = int(rng.choice([1, 2, 8, 33, 256, 1024]))
            B = int(rng.choice([1, 2, 16, 64, 128, 3]))
            ids = rng.integers(-2, E + 3, size=(T, K)).astype(np.int32)      # some out of range
            cases.append((ids, E, B))
    # single- / multi-workgroup threshold: S = 4096 and 4097 slots
    cases.append((rng.integers(0, 64, size=(4096, 1)).astype(np.int32), 64, 16))
    cases.append((rng.integers(0, 64, size=(4097, 1)).astype(np.int32), 64, 16))
    # every id out of range; one expert takes everything; max experts
    cases.append((np.full((300, 4), 9, np.int32), 8, 16))
    cases.append((np.zeros((50000, 2), np.int32), 4, 64))
    cases.append((rng.integers(0, 1024, size=(30000, 8)).astype(np.int32), 1024, 32))
    for n, (ids, E, B) in enumerate(cases):
        run_and_compare(ids, E, B, f"case {n}")


def test_align_is_deterministic():
    ids_np = ms.zipf_topk_ids(1, ms.TAG_IDS, 16384, 8, 256, 1.1)
    dev = device()
    ids = torch.from_numpy(ids_np).to(dev)
    first = moe.moe_align_sort(ids, 256, 64)["sorted_token_ids"].clone()
    for _ in range(10):
        again = moe.moe_align_sort(ids, 256, 64)["sorted_token_ids"]
        assert torch.equal(first, again)


def test_align_many_experts_large():
    # 4M slots over 1024 experts: the widest chunk that 1024 experts leave room for
    rng = np.random.default_rng(11)
    run_and_compare(rng.integers(0, 1024, size=(524288, 8)).astype(np.int32), 1024, 32, "524288x8/1024")


def test_align_workspace_reused_across_paths():
    # one zeroed workspace serves calls of every path in stream order: the
    # single workgroup, one launch with the merge, one launch with the column
    # scans and two barriers, and the count/scan/place launches; the barrier
    # words are zero again after each call and no wait gave up
    dev = device()
    shapes = [(16384, 8, 256, 64), (100, 8, 64, 16), (131072, 8, 256, 64), (1024, 8, 256, 64),
              (5000, 1, 3, 1), (1_200_000, 8, 256, 64), (16384, 8, 256, 128), (40000, 8, 1024, 32)]
    need = max(moe.moe_align_sort_workspace_bytes(T, K, E, B) for T, K, E, B in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for T, K, E, B in shapes:
        ids_np = ms.zipf_topk_ids(T, ms.TAG_IDS, T, K, E, 1.1)
        ids = torch.from_numpy(ids_np).to(dev)
        r = moe.moe_align_sort(ids, E, B, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.align_sort(ids_np, E, B)
        assert np.array_equal(r["sorted_token_ids"].cpu().numpy(), ref["sorted_token_ids"]), (T, K, E, B)
        assert np.array_equal(r["expert_ids"].cpu().numpy(), ref["expert_ids"]), (T, K, E, B)
        words = ws[:4352].view(torch.int32).cpu().numpy()
        counters = np.concatenate([words[[0, 32]], words[64:576:32]])   # status, top, 16 groups
        assert (counters == 0).all(), (T, K, E, B, counters)    # reset by every call; status 0
        say(f"shared workspace T={T} K={K} E={E} B={B}: bit-exact, counters zero, "
            f"generations {words[576:1088:32][:4].tolist()}...")


@pytest.mark.parametrize("E", [700, 800])
def test_align_mask_and_ballot_ranks_near_the_lds_limit(E):
    # 700 experts still rank with per-wave LDS masks, 800 with ballots
    rng = np.random.default_rng(E)
    run_and_compare(rng.integers(0, E, size=(300000, 8)).astype(np.int32), E, 64, f"300000x8/{E}")


def test_align_beyond_one_resident_round():
    # 9.6M slots need more than 256 chunks of 32768: counts, column scans and
    # placement in three launches
    ids = ms.zipf_topk_ids(3, ms.TAG_IDS, 1_200_000, 8, 256, 1.1)
    run_and_compare(ids, 256, 64, "1200000x8/256")


def test_align_tagged_merge_calls_in_a_row():
    # 8 and 16 workgroups merge tagged count words without a grid barrier:
    # calls of different shapes in a row on one workspace (the 16-workgroup
    # rows 8..15 still hold the first call's words when the third call reads
    # them), mixed with calls that write plain counts into the same region
    dev = device()
    shapes = [(2500, 8, 256, 64), (1024, 8, 256, 16), (2500, 8, 256, 64), (131072, 8, 256, 64),
              (2100, 8, 200, 32), (600, 8, 32, 1), (2500, 8, 256, 64)]
    need = max(moe.moe_align_sort_workspace_bytes(T, K, E, B) for T, K, E, B in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for n, (T, K, E, B) in enumerate(shapes):
        ids_np = ms.zipf_topk_ids(100 + n, ms.TAG_IDS, T, K, E, 1.1)
        ids = torch.from_numpy(ids_np).to(dev)
        r = moe.moe_align_sort(ids, E, B, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.align_sort(ids_np, E, B)
        assert np.array_equal(r["sorted_token_ids"].cpu().numpy(), ref["sorted_token_ids"]), (n, T, K, E, B)
        assert np.array_equal(r["expert_ids"].cpu().numpy(), ref["expert_ids"]), (n, T, K, E, B)
        assert int(ws[:4].view(torch.int32).item()) == 0, (n, "a wait gave up")
        say(f"tagged merge call {n}: T={T} K={K} E={E} B={B} bit-exact")
