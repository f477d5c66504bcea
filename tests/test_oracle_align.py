"""Pins for the oracle's Align & Sort (a stable counting sort with per-expert
padding to whole blocks of block_size_m).

* exhaustive brute force on every tiny id table against a different algorithm
  (filter the slots expert by expert, then pad);
* block size 1 reduces to numpy's stable argsort;
* closed forms and invariants at the align-only workload's full size
  (16384 tokens x top-8 of 256 experts, Zipf(1.1), block 64);
* capacity is the exact maximum of the padded length;
* a small table worked out by hand.
"""
import itertools

import numpy as np
import pytest

import moe_synth as ms
import oracle


def brute_align(ids: np.ndarray, E: int, B: int):
    """Filter-per-expert: for e = 0..E-1 collect slot indices i (ascending) with
    ids[i] == e, pad the run with the sentinel S up to a multiple of B."""
    flat = ids.ravel()
    S = flat.size
    out, blocks = [], []
    for e in range(E):
        run = [i for i in range(S) if flat[i] == e]
        if not run:
            continue
        nb = -(-len(run) // B)
        run += [S] * (nb * B - len(run))
        out += run
        blocks += [e] * nb
    return out, blocks


def check_against_brute(ids, E, B):
    r = oracle.align_sort(ids, E, B)
    out, blocks = brute_align(ids, E, B)
    S = ids.size
    C = oracle.align_capacity(S, E, B)
    P = len(out)
    assert r["num_tokens_post_padded"] == P
    want_sorted = np.array(out + [S] * (C - P), np.int32)
    want_blocks = np.array(blocks + [-1] * (C // B - len(blocks)), np.int32)
    assert np.array_equal(r["sorted_token_ids"], want_sorted)
    assert np.array_equal(r["expert_ids"], want_blocks)


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_exhaustive_tiny_tables(B):
    n = 0
    for E in (1, 2, 3):
        for T in (0, 1, 2, 3):
            for K in (1, 2):
                if T * K > 4:
                    continue
                for flat in itertools.product(range(-1, E + 1), repeat=T * K):
                    ids = np.array(flat, np.int32).reshape(T, K)
                    check_against_brute(ids, E, B)
                    n += 1
    assert n > 500


def test_random_small_tables():
    rng = np.random.default_rng(0)
    for _ in range(200):
        E = int(rng.integers(1, 40))
        T = int(rng.integers(0, 60))
        K = int(rng.integers(1, 5))
        B = int(rng.choice([1, 2, 4, 8, 16, 5]))
        ids = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        check_against_brute(ids, E, B)


def test_block_one_is_stable_argsort():
    rng = np.random.default_rng(2)
    for E in (1, 7, 256):
        ids = rng.integers(0, E, size=(500, 3)).astype(np.int32)
        r = oracle.align_sort(ids, E, 1)
        S = ids.size
        assert r["num_tokens_post_padded"] == S
        assert np.array_equal(r["sorted_token_ids"][:S], np.argsort(ids.ravel(), kind="stable"))
        assert np.array_equal(r["expert_ids"][:S], np.sort(ids.ravel()))


def test_hand_worked_example():
    # ids (T=3, K=2): slots 0..5 -> experts 2,0 | 1,2 | 0,3 ; E=4, B=2.
    # counts: e0 {1,4}, e1 {2}, e2 {0,3}, e3 {5}; padded 2,2,2,2 -> P = 8.
    # capacity: S=6, min(E,S)=4 -> 2*floor((6+4*1)/2) = 10.
    ids = np.array([[2, 0], [1, 2], [0, 3]], np.int32)
    r = oracle.align_sort(ids, 4, 2)
    assert r["num_tokens_post_padded"] == 8
    assert r["sorted_token_ids"].tolist() == [1, 4, 2, 6, 0, 3, 5, 6, 6, 6]
    assert r["expert_ids"].tolist() == [0, 1, 2, 3, -1]
    assert r["expert_offsets"].tolist() == [0, 2, 4, 6, 8]


def test_capacity_is_exact_maximum():
    for S in range(0, 9):
        for E in range(1, 6):
            for B in (1, 2, 3, 4):
                best = 0
                # every way to spread S slots over E experts (compositions)
                for cut in itertools.product(range(S + 1), repeat=E - 1):
                    if sum(cut) > S:
                        continue
                    cnt = list(cut) + [S - sum(cut)]
                    best = max(best, sum(-(-c // B) * B for c in cnt))
                assert oracle.align_capacity(S, E, B) == best, (S, E, B)


def test_invariants_full_align_workload():
    cfg = ms.CONFIGS["align_16k"]
    ids = ms.zipf_topk_ids(0, ms.TAG_IDS, cfg["T"], cfg["K"], cfg["E"], cfg["zipf_s"])
    E, B = cfg["E"], cfg["B"]
    r = oracle.align_sort(ids, E, B)
    S = ids.size
    srt, blk, P, off = (r["sorted_token_ids"], r["expert_ids"], r["num_tokens_post_padded"],
                        r["expert_offsets"])
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert P == int(np.sum(-(-cnt // B) * B))
    assert len(srt) == oracle.align_capacity(S, E, B)
    real = srt[srt != S]
    assert np.array_equal(np.sort(real), np.arange(S))            # a permutation of the slots
    assert np.all(srt[P:] == S)
    assert np.all(np.diff(off) % B == 0)
    used = blk[:P // B]
    assert np.all(np.diff(used) > 0) or np.all(np.diff(used) >= 0)
    assert np.all(blk[P // B:] == -1)
    flat = ids.ravel()
    for j in range(P // B):
        rows = srt[j * B:(j + 1) * B]
        rows = rows[rows != S]
        assert np.all(flat[rows] == blk[j])
        assert np.all(np.diff(rows) > 0)                           # stable within the block
    for e in range(E):
        seg = srt[off[e]:off[e + 1]]
        assert np.array_equal(seg[:cnt[e]], np.flatnonzero(flat == e))
