"""Pins for the oracle's top-k routing.

* no bias, no groups: softmax and the sigmoid are increasing in the logit, so
  the chosen experts are numpy's top-K of the logits (a library routine);
* closed forms for the weights: softmax ratios are exp of logit differences,
  sigmoid(0) = 1/2 and sigmoid(l) + sigmoid(-l) = 1, renormalised weights sum
  to one, routed_scaling scales linearly;
* a dominant bias forces its experts in while the weights stay unbiased;
* group-limited selection against brute-force enumeration of every group
  subset and every expert subset;
* equal keys go to the lower expert id.
"""
import itertools

import numpy as np

import oracle


def test_topk_equals_argsort_of_logits():
    rng = np.random.default_rng(0)
    for score in ("softmax", "sigmoid"):
        for E, K in ((8, 2), (32, 4), (64, 8)):
            logits = rng.normal(0, 1.5, size=(200, E)).astype(np.float32)
            ids, _ = oracle.route_topk(logits, K, score=score)
            want = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :K]
            assert np.array_equal(ids, want), (score, E, K)


def test_softmax_weight_closed_forms():
    rng = np.random.default_rng(1)
    logits = rng.normal(0, 1, size=(100, 16)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 4, score="softmax", renormalize=True)
    l = logits.astype(np.float64)
    lk = np.take_along_axis(l, ids, axis=1)
    ratio = w[:, 1:].astype(np.float64) / w[:, :1]
    assert np.allclose(ratio, np.exp(lk[:, 1:] - lk[:, :1]), rtol=3e-7)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=4e-7)
    # K = E without renormalisation: all E softmax values, descending, sum 1
    ids, w = oracle.route_topk(logits, 16, score="softmax", renormalize=False)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    # routed_scaling multiplies
    _, w1 = oracle.route_topk(logits, 4, score="softmax", renormalize=True, routed_scaling=2.5)
    _, w0 = oracle.route_topk(logits, 4, score="softmax", renormalize=True)
    assert np.allclose(w1, 2.5 * w0.astype(np.float64), rtol=1e-7)


def test_sigmoid_closed_forms():
    logits = np.array([[0.0, -50.0, -60.0], [2.0, -70.0, -80.0], [-2.0, -90.0, -99.0]], np.float32)
    ids, w = oracle.route_topk(logits, 1, score="sigmoid", renormalize=False)
    assert ids[:, 0].tolist() == [0, 0, 0]
    assert w[0, 0] == np.float32(0.5)
    assert abs(float(w[1, 0]) + float(w[2, 0]) - 1.0) < 1e-7
    assert abs(float(w[1, 0]) - 0.8807970779778823) < 1e-7


def test_bias_selects_but_weights_stay_unbiased():
    rng = np.random.default_rng(3)
    E, K = 32, 4
    logits = rng.normal(0, 1, size=(50, E)).astype(np.float32)
    forced = rng.choice(E, size=K, replace=False)
    bias = np.zeros(E, np.float32)
    bias[forced] = 10.0
    ids, w = oracle.route_topk(logits, K, score="sigmoid", bias=bias, renormalize=False)
    for t in range(50):
        assert set(ids[t]) == set(forced.tolist())
    sig = 1.0 / (1.0 + np.exp(-np.take_along_axis(logits.astype(np.float64), ids, axis=1)))
    assert np.allclose(w, sig, rtol=1e-7)
    # the forced experts come out in descending order of their scores
    assert np.all(np.diff(w, axis=1) <= 0)


def test_ties_go_to_lower_id():
    logits = np.zeros((3, 10), np.float32)
    ids, w = oracle.route_topk(logits, 3, score="softmax")
    assert ids.tolist() == [[0, 1, 2]] * 3
    assert np.allclose(w, 1 / 3)
    logits[1, 7] = 1.0
    ids, _ = oracle.route_topk(logits, 3, score="sigmoid")
    assert ids[1].tolist() == [7, 0, 1]


def _keys_f32(logits, bias):
    s = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    return s + bias if bias is not None else s


def test_group_limited_selection_brute_force():
    rng = np.random.default_rng(4)
    E, n_group, topk_group, K = 12, 4, 2, 3
    gsize = E // n_group
    for trial in range(300):
        logits = rng.normal(0, 2, size=(1, E)).astype(np.float32)
        bias = rng.uniform(-0.1, 0.1, size=E).astype(np.float32)
        ids, w = oracle.route_topk(logits, K, score="sigmoid", bias=bias, n_group=n_group,
                                   topk_group=topk_group, renormalize=True)
        key = _keys_f32(logits[0], bias)
        gscore = [np.float32(np.sort(key[g * gsize:(g + 1) * gsize])[-2:].astype(np.float32).sum(
            dtype=np.float32)) for g in range(n_group)]
        # best group subset: largest total group score; ties -> lexicographically smaller
        best_g = max(itertools.combinations(range(n_group), topk_group),
                     key=lambda c: (sorted([gscore[g] for g in c], reverse=True),
                                    [-g for g in c]))
        allowed = [e for e in range(E) if e // gsize in best_g]
        best_e = max(itertools.combinations(allowed, K),
                     key=lambda c: (sorted([key[e] for e in c], reverse=True), [-e for e in c]))
        order = sorted(best_e, key=lambda e: (-key[e], e))
        assert ids[0].tolist() == order, trial
        s = 1.0 / (1.0 + np.exp(-logits[0].astype(np.float64)[order]))
        assert np.allclose(w[0], s / s.sum(), rtol=1e-7)


def test_append_shared_column():
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 1, size=(7, 8)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 2, score="softmax", append_shared=True)
    ids0, w0 = oracle.route_topk(logits, 2, score="softmax")
    assert ids.shape == (7, 3)
    assert np.array_equal(ids[:, :2], ids0) and np.array_equal(w[:, :2], w0)
    assert np.all(ids[:, 2] == 8) and np.all(w[:, 2] == 1.0)
