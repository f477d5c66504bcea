"""Pins of the oracle's permute / unpermute functions (no GPU).

The permute moves token rows into Align & Sort's padded expert order and
records the inverse map; unpermute-combine is the weighted combine read back
through that map.  They are checked against a table worked by hand, a round
trip, the (separately pinned) combine and Align & Sort invariants."""
import numpy as np
import pytest

import oracle


def test_hand_worked_table():
    # ids [[1,0],[1,2],[0,1]], E = 3, B = 2.  Slots 0..5 go to experts
    # 1,0,1,2,0,1.  Expert 0 holds slots 1,4 (2 rows), expert 1 slots 0,2,5
    # (padded to 4), expert 2 slot 3 (padded to 2): P = 8, sentinel 6.
    ids = np.array([[1, 0], [1, 2], [0, 1]], np.int32)
    al = oracle.align_sort(ids, 3, 2)
    assert list(al["sorted_token_ids"]) == [1, 4, 0, 2, 5, 6, 3, 6]
    x = np.array([[10, 11], [20, 21], [30, 31]], np.int16)      # token t's row
    xp = oracle.permute_rows(x, al["sorted_token_ids"], 2)
    want = [[10, 11], [30, 31], [10, 11], [20, 21], [30, 31], [0, 0], [20, 21], [0, 0]]
    assert xp.tolist() == want
    assert list(oracle.row_of_slot(al["sorted_token_ids"], 6)) == [2, 0, 3, 6, 1, 4]


def random_case(rng, T, K, E, B, p_invalid=0.1):
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    bad = rng.random((T, K)) < p_invalid
    ids[bad] = rng.choice([-1, E, E + 3], size=int(bad.sum()))
    return ids, oracle.align_sort(ids, E, B)


@pytest.mark.parametrize("T,K,E,B", [(1, 1, 1, 1), (7, 3, 5, 4), (64, 8, 16, 16), (200, 2, 33, 32)])
def test_row_of_slot_inverts_the_layout(T, K, E, B):
    rng = np.random.default_rng(T * 131 + K)
    ids, al = random_case(rng, T, K, E, B)
    S = T * K
    srt = al["sorted_token_ids"]
    ros = oracle.row_of_slot(srt, S)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(ros < 0, ~valid)                 # -1 exactly on skipped slots
    assert np.array_equal(srt[ros[valid]], np.nonzero(valid)[0])
    # each placed row sits in a block of its slot's expert
    P = al["num_tokens_post_padded"]
    rows = ros[valid]
    assert (rows < P).all()
    assert np.array_equal(al["expert_ids"][rows // B], flat[valid])


@pytest.mark.parametrize("T,K,E,B", [(5, 1, 3, 2), (64, 1, 8, 16), (300, 1, 32, 64)])
def test_round_trip_with_unit_weights(T, K, E, B):
    rng = np.random.default_rng(T)
    ids, al = random_case(rng, T, K, E, B)
    x = rng.standard_normal((T, 24)).astype(np.float32)
    xp = oracle.permute_rows(x, al["sorted_token_ids"], K)
    ros = oracle.row_of_slot(al["sorted_token_ids"], T * K)
    back = oracle.unpermute_combine(xp, np.ones((T, K), np.float32), ros)
    valid = ((ids >= 0) & (ids < E)).ravel()
    assert np.array_equal(back[valid], x[valid].astype(np.float64))
    assert not back[~valid].any()
    # padding rows of the permuted buffer are zero, and only they are
    placed = al["sorted_token_ids"] < T * K
    assert not xp[~placed].any()


@pytest.mark.parametrize("T,K,E,B", [(9, 4, 6, 4), (128, 8, 32, 16), (50, 3, 7, 1)])
def test_unpermute_combine_equals_combine(T, K, E, B):
    rng = np.random.default_rng(K * 977 + T)
    ids, al = random_case(rng, T, K, E, B)
    H = 40
    y_slots = rng.standard_normal((T * K, H)).astype(np.float32)
    w = rng.random((T, K)).astype(np.float32)
    # slot-indexed rows moved into the padded layout (one row per slot: K = 1)
    y_perm = oracle.permute_rows(y_slots, al["sorted_token_ids"], 1)
    ros = oracle.row_of_slot(al["sorted_token_ids"], T * K)
    got = oracle.unpermute_combine(y_perm, w, ros)
    want = oracle.combine(y_slots, w, ids, E)
    assert np.array_equal(got, want)                      # same sums in the same order


def test_permute_moves_bytes_of_any_width():
    rng = np.random.default_rng(3)
    ids, al = random_case(rng, 33, 2, 4, 8, 0.0)
    for dt, w in ((np.uint8, 48), (np.uint16, 7168), (np.float32, 5)):
        x = rng.integers(0, 200, (33, w)).astype(dt)
        xp = oracle.permute_rows(x, al["sorted_token_ids"], 2)
        placed = al["sorted_token_ids"] < 66
        assert np.array_equal(xp[placed], x[al["sorted_token_ids"][placed] // 2])


def test_rows_past_the_padded_count_are_left_alone():
    rng = np.random.default_rng(11)
    ids, al = random_case(rng, 40, 2, 16, 8, 0.0)
    srt, P = al["sorted_token_ids"], al["num_tokens_post_padded"]
    C = srt.shape[0]
    assert P < C
    x = rng.integers(1, 200, (40, 32)).astype(np.uint8)
    before = np.full((C, 32), 0xAB, np.uint8)
    xp = oracle.permute_rows(x, srt, 2, P=P, out=before)
    assert (xp[P:] == 0xAB).all()
    full = oracle.permute_rows(x, srt, 2)
    assert np.array_equal(xp[:P], full[:P])
    assert not full[P:].any()


# ----------------------------------------------- gradient of the unpermute --
def test_unpermute_backward_hand_worked():
    # The layout of the hand-worked table: rows [1,4,0,2,5,6,3,6] hold slots
    # (6 = padding).  Token t's slots are 2t, 2t+1.
    ids = np.array([[1, 0], [1, 2], [0, 1]], np.int32)
    srt = oracle.align_sort(ids, 3, 2)["sorted_token_ids"]
    w = np.array([[0.5, 2.0], [1.0, -1.0], [0.25, 4.0]], np.float32)
    g = np.array([[1, 2], [3, 4], [5, 6]], np.float32)              # d_out[t]
    y = np.arange(16, dtype=np.float32).reshape(8, 2)               # y_perm rows
    dy, dw = oracle.unpermute_combine_backward(g, y, w, srt)
    # row r holds slot s: d_y = w[s] * d_out[s // 2]
    want = [[2.0 * 1, 2.0 * 2], [0.25 * 5, 0.25 * 6], [0.5 * 1, 0.5 * 2], [1.0 * 3, 1.0 * 4],
            [4.0 * 5, 4.0 * 6], [0, 0], [-1.0 * 3, -1.0 * 4], [0, 0]]
    assert dy.tolist() == want
    # slot s: <d_out[s // 2], y[row of s]>, rows of slots 0..5 = [2,0,3,6,1,4]
    rows = [2, 0, 3, 6, 1, 4]
    want_w = [float(g[s // 2] @ y[rows[s]]) for s in range(6)]
    assert dw.ravel().tolist() == want_w


@pytest.mark.parametrize("T,K,E,B", [(7, 3, 5, 4), (64, 8, 16, 16), (200, 2, 33, 32)])
def test_unpermute_backward_is_the_adjoint(T, K, E, B):
    # unpermute_combine is linear in y_perm and in w: for any directions,
    # <d_out, UC(dY, w)> = <d_y_perm, dY> and <d_out, UC(y, dW)> = <d_w, dW>,
    # with UC the separately pinned forward.
    rng = np.random.default_rng(T + 7 * K)
    ids, al = random_case(rng, T, K, E, B)
    srt, P = al["sorted_token_ids"], al["num_tokens_post_padded"]
    H = 12
    C = srt.shape[0]
    ros = oracle.row_of_slot(srt, T * K)
    w = rng.standard_normal((T, K)).astype(np.float32)
    g = rng.standard_normal((T, H)).astype(np.float32)
    y = rng.standard_normal((C, H)).astype(np.float32)
    dy, dw = oracle.unpermute_combine_backward(g, y, w, srt, P=P)
    dY = rng.standard_normal((C, H)).astype(np.float32)
    lhs = float(np.sum(g.astype(np.float64) * oracle.unpermute_combine(dY, w, ros)))
    rhs = float(np.sum(dy * dY[:P].astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * H * K
    dW = rng.standard_normal((T, K)).astype(np.float32)
    lhs = float(np.sum(g.astype(np.float64) * oracle.unpermute_combine(y, dW, ros)))
    rhs = float(np.sum(dw * dW.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)) * H * K
    # padding rows get no gradient; skipped slots get a zero weight gradient
    pad = srt[:P] >= T * K
    assert (dy[pad] == 0).all()
    assert (dw.ravel()[ros < 0] == 0).all()


def _bf16_rne(v32):
    # round-to-nearest-even on the bit pattern (add 0x7FFF plus the kept lsb)
    u = v32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32)


def test_unpermute_backward_rounding_of_the_delivered_rows():
    rng = np.random.default_rng(3)
    ids, al = random_case(rng, 40, 4, 6, 8, p_invalid=0.0)
    srt, P = al["sorted_token_ids"], al["num_tokens_post_padded"]
    w = rng.standard_normal((40, 4)).astype(np.float32)
    g = rng.standard_normal((40, 16)).astype(np.float32)
    y = rng.standard_normal((srt.shape[0], 16)).astype(np.float32)
    exact, _ = oracle.unpermute_combine_backward(g, y, w, srt, P=P)
    f32, _ = oracle.unpermute_combine_backward(g, y, w, srt, P=P, round_to="f32")
    b16, _ = oracle.unpermute_combine_backward(g, y, w, srt, P=P, round_to="bf16")
    ref32 = exact.astype(np.float32)                # a product of two floats is exact in double
    assert np.array_equal(f32, ref32.astype(np.float64))
    assert np.array_equal(b16, _bf16_rne(ref32).astype(np.float64))
