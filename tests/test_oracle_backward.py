"""Pins of the oracle's backward (no GPU).

The backward is the derivative of the forward, so it is checked against
central finite differences of the forward oracle (itself pinned elsewhere),
and, for one expert with weight 1, against the textbook SwiGLU backward in
matrix form (numpy float64)."""
import numpy as np
import pytest

import oracle


def tiny(seed, T=5, K=2, E=3, H=8, I=6, invalid=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (0.4 * rng.standard_normal((E, 2 * I, H))).astype(np.float32)
    w2 = (0.4 * rng.standard_normal((E, H, I))).astype(np.float32)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    if invalid:
        ids[1, 0] = -1                       # a skipped slot
    w = rng.random((T, K)).astype(np.float32)
    d_out = rng.standard_normal((T, H)).astype(np.float32)
    return x, w13, w2, ids, w, d_out


def loss(x, w13, w2, ids, w, d_out):
    out, _ = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64", E=w13.shape[0])
    return float((out * d_out.astype(np.float64)).sum())


def fd(fn, arr, idx, eps=2.0 ** -8):
    a = arr.copy(); a[idx] += eps; up = float(a[idx]) - float(arr[idx]); lp = fn(a)
    b = arr.copy(); b[idx] -= eps; dn = float(arr[idx]) - float(b[idx]); lm = fn(b)
    return (lp - lm) / (up + dn)


@pytest.mark.parametrize("seed", [0, 1])
def test_ffn_backward_matches_finite_differences(seed):
    x, w13, w2, ids, w, d_out = tiny(seed)
    _, y = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64", E=3)
    dx, dw13, dw2, dwk = oracle.ffn_backward(x, w13, w2, ids, w, y, d_out, w_dtype="f32",
                                             x_dtype="f32", inter="f64")
    rng = np.random.default_rng(100 + seed)
    checks = []
    for _ in range(8):
        i = tuple(rng.integers(0, s) for s in x.shape)
        checks.append((dx[i], fd(lambda a: loss(a, w13, w2, ids, w, d_out), x, i)))
        i = tuple(rng.integers(0, s) for s in w13.shape)
        checks.append((dw13[i], fd(lambda a: loss(x, a, w2, ids, w, d_out), w13, i)))
        i = tuple(rng.integers(0, s) for s in w2.shape)
        checks.append((dw2[i], fd(lambda a: loss(x, w13, a, ids, w, d_out), w2, i)))
        i = tuple(rng.integers(0, s) for s in w.shape)
        checks.append((dwk[i], fd(lambda a: loss(x, w13, w2, ids, a, d_out), w, i)))
    got = np.array([c[0] for c in checks])
    want = np.array([c[1] for c in checks])
    scale = np.abs(want).max()
    assert np.abs(got - want).max() <= 2e-3 * scale, np.abs(got - want).max() / scale
    # the skipped slot has no weight gradient
    assert dwk[1, 0] == 0.0


def test_single_expert_is_the_textbook_swiglu_backward():
    rng = np.random.default_rng(7)
    T, H, I = 9, 12, 10
    X = rng.standard_normal((T, H))
    Wg, Wu = rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3
    Wd = rng.standard_normal((H, I)) * 0.3
    dY = rng.standard_normal((T, H))
    # the oracle on the same fp32 values
    x32, w13 = X.astype(np.float32), np.concatenate([Wg, Wu])[None].astype(np.float32)
    w2 = Wd[None].astype(np.float32)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    _, y = oracle.moe_layer(x32, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64", E=1)
    dx, dw13, dw2, _ = oracle.ffn_backward(x32, w13, w2, ids, w, y, dY.astype(np.float32),
                                           w_dtype="f32", x_dtype="f32", inter="f64")
    X, Wg, Wu, Wd = (np.float64(v) for v in (x32, w13[0, :I], w13[0, I:], w2[0]))
    dY = np.float64(dY.astype(np.float32))
    G, U = X @ Wg.T, X @ Wu.T
    S = 1.0 / (1.0 + np.exp(-G))
    A = G * S * U
    dA = dY @ Wd
    dG = dA * U * (S + G * S * (1.0 - S))
    dU = dA * G * S
    np.testing.assert_allclose(dw2[0], dY.T @ A, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw13[0], np.concatenate([dG.T @ X, dU.T @ X]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dx, dG @ Wg + dU @ Wu, rtol=1e-10, atol=1e-12)


def test_rounded_intermediate_enters_the_down_weight_gradient():
    x, w13, w2, ids, w, d_out = tiny(3, invalid=False)
    _, y = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64", E=3)
    g64 = oracle.ffn_backward(x, w13, w2, ids, w, y, d_out, w_dtype="f32", x_dtype="f32", inter="f64")
    g16 = oracle.ffn_backward(x, w13, w2, ids, w, y, d_out, w_dtype="f32", x_dtype="f32", inter="bf16")
    assert not np.array_equal(g64[2], g16[2])
    # only dW2 sees the rounding (straight-through elsewhere)
    for a, b in zip((g64[0], g64[1], g64[3]), (g16[0], g16[1], g16[3])):
        assert np.array_equal(a, b)
    np.testing.assert_allclose(g16[2], g64[2], rtol=2e-2, atol=2e-2 * np.abs(g64[2]).max())


@pytest.mark.parametrize("score,renorm,scaling,groups", [("softmax", True, 1.0, 1), ("softmax", False, 1.0, 1),
                                                          ("sigmoid", True, 2.5, 2), ("sigmoid", False, 1.0, 1)])
def test_route_backward_matches_finite_differences(score, renorm, scaling, groups):
    rng = np.random.default_rng(11)
    T, E, K = 6, 8, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(T):                       # clear margins: the choice survives a perturbation
        logits[t, rng.choice(E, K, replace=False)] += 3.0
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32) if groups > 1 else None
    kw = dict(score=score, renormalize=renorm, routed_scaling=scaling, n_group=groups,
              topk_group=groups if groups == 1 else 2, bias=bias)
    ids, w = oracle.route_topk(logits, K, **kw)
    d_w = rng.standard_normal((T, K)).astype(np.float32)

    dmap = np.zeros((T, E))                  # the upstream gradient keyed by expert, not column
    for t in range(T):
        dmap[t, ids[t]] = d_w[t]

    def L(lg):
        ids2, w2 = oracle.route_topk(lg, K, **kw)
        assert (np.sort(ids2, 1) == np.sort(ids, 1)).all()    # the same experts (order may swap)
        return float(sum(w2[t, k] * dmap[t, ids2[t, k]] for t in range(T) for k in range(K)))

    dl = oracle.route_backward(logits, ids, d_w, K, score=score, renormalize=renorm, routed_scaling=scaling)
    got, want = [], []
    for t in range(T):
        for e in range(E):
            got.append(dl[t, e])
            want.append(fd(L, logits, (t, e), eps=2.0 ** -10))
    got, want = np.array(got), np.array(want)
    assert np.abs(got - want).max() <= 2e-3 * np.abs(want).max()


def test_route_backward_ignores_the_shared_column():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((4, 6)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 2, score="softmax", append_shared=True)
    d_w = rng.standard_normal((4, 3)).astype(np.float32)
    a = oracle.route_backward(logits, ids, d_w, 2, score="softmax", append_shared=True)
    d_w[:, 2] = 100.0
    b = oracle.route_backward(logits, ids, d_w, 2, score="softmax", append_shared=True)
    assert np.array_equal(a, b)
