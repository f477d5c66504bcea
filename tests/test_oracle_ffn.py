"""Pins for the oracle's expert FFN, per-token fp8 quantisation and combine.

* the dense formulation out = sum_e G[t,e] FFN_e(x_t), computed expert-major
  with numpy float64 matmuls over all tokens (a different loop order and a
  library routine), equals the oracle's per-token loop;
* a single expert with weight 1 is the textbook SwiGLU FFN;
* linearity in the routing weights, identical experts, skipped ids, the
  appended shared expert;
* the bf16 / fp32 / fp8 rounding hooks against the same dense formulation with
  torch's own casts applied to the intermediate;
* the per-token E4M3 quantisation against its error bound and torch's cast.
"""
import numpy as np
import torch

import oracle


def silu(g):
    return g / (1.0 + np.exp(-g))


def dense_layer(x, w13, w2, ids, w, E, round_a=None):
    """Expert-major dense formulation in float64."""
    T, H = x.shape
    I = w13.shape[1] // 2
    K = ids.shape[1]
    G = np.zeros((T, E))
    for k in range(K):
        ok = (ids[:, k] >= 0) & (ids[:, k] < E)
        np.add.at(G, (np.flatnonzero(ok), ids[ok, k]), w[ok, k].astype(np.float64))
    out = np.zeros((T, H))
    for e in range(E):
        a = silu(x @ w13[e, :I].T) * (x @ w13[e, I:].T)        # [T, I]
        if round_a is not None:
            a = round_a(a)
        out += G[:, e:e + 1] * (a @ w2[e].T)
    return out


def rand_problem(rng, T=24, H=32, I=48, E=5, K=2):
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    w13 = rng.normal(0, 0.2, (E, 2 * I, H)).astype(np.float32)
    w2 = rng.normal(0, 0.2, (E, H, I)).astype(np.float32)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    return x, w13, w2, ids, w


def test_dense_formulation_fp64():
    rng = np.random.default_rng(0)
    x, w13, w2, ids, w = rand_problem(rng)
    out, _ = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64")
    ref = dense_layer(x.astype(np.float64), w13.astype(np.float64), w2.astype(np.float64), ids, w, 5)
    # y_slots are stored as fp32, so agreement is at fp32 resolution of each slot
    assert np.max(np.abs(out - ref)) <= 2e-7 * np.max(np.abs(ref))


def test_single_expert_textbook_ffn():
    rng = np.random.default_rng(1)
    T, H, I = 9, 16, 20
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    wg = rng.normal(0, 0.3, (I, H)); wu = rng.normal(0, 0.3, (I, H)); wd = rng.normal(0, 0.3, (H, I))
    w13 = np.concatenate([wg, wu])[None].astype(np.float32)
    w2 = wd[None].astype(np.float32)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out, y = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f64")
    xd = x.astype(np.float64)
    g = xd @ w13[0, :I].astype(np.float64).T
    u = xd @ w13[0, I:].astype(np.float64).T
    ref = ((g * (1 / (1 + np.exp(-g)))) * u) @ w2[0].astype(np.float64).T
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())
    assert np.array_equal(out, y.astype(np.float64))


def test_linearity_identical_experts_skips_and_shared():
    rng = np.random.default_rng(2)
    x, w13, w2, ids, w = rand_problem(rng, E=4, K=3)
    E = 4
    base, y = oracle.moe_layer(x, w13, w2, ids, w, w_dtype="f32", x_dtype="f32", inter="f32")
    twice, _ = oracle.moe_layer(x, w13, w2, ids, 2 * w, w_dtype="f32", x_dtype="f32", inter="f32")
    assert np.array_equal(twice, 2 * base)
    # identical experts: out = (sum_k w_k) * FFN(x)
    w13s = np.repeat(w13[:1], E, 0); w2s = np.repeat(w2[:1], E, 0)
    same, ys = oracle.moe_layer(x, w13s, w2s, ids, w, w_dtype="f32", x_dtype="f32", inter="f32")
    one, _ = oracle.moe_layer(x, w13[:1], w2[:1], np.zeros((x.shape[0], 1), np.int32),
                              np.ones((x.shape[0], 1), np.float32), w_dtype="f32", x_dtype="f32",
                              inter="f32")
    assert np.allclose(same, w.sum(1, dtype=np.float64)[:, None] * one, rtol=1e-12, atol=1e-15)
    # ids out of range are skipped: same as giving those slots weight 0
    bad = ids.copy(); bad[::3, 1] = -1; bad[1::4, 2] = E
    wz = w.copy(); wz[bad < 0] = 0; wz[bad >= E] = 0
    skip, yb = oracle.moe_layer(x, w13, w2, bad, w, w_dtype="f32", x_dtype="f32", inter="f32")
    zero, _ = oracle.moe_layer(x, w13, w2, ids, wz, w_dtype="f32", x_dtype="f32", inter="f32")
    assert np.array_equal(skip, zero)
    assert np.all(yb[(bad.ravel() < 0) | (bad.ravel() >= E)] == 0)
    # the appended shared expert (id E, weight 1) adds its FFN
    w13x = np.concatenate([w13, rng.normal(0, .2, (1,) + w13.shape[1:]).astype(np.float32)])
    w2x = np.concatenate([w2, rng.normal(0, .2, (1,) + w2.shape[1:]).astype(np.float32)])
    ids_s = np.concatenate([ids, np.full((ids.shape[0], 1), E, np.int32)], 1)
    w_s = np.concatenate([w, np.ones((w.shape[0], 1), np.float32)], 1)
    with_s, _ = oracle.moe_layer(x, w13x, w2x, ids_s, w_s, w_dtype="f32", x_dtype="f32", inter="f32")
    sh, _ = oracle.moe_layer(x, w13x[E:], w2x[E:], np.zeros((x.shape[0], 1), np.int32),
                             np.ones((x.shape[0], 1), np.float32), w_dtype="f32", x_dtype="f32",
                             inter="f32")
    assert np.allclose(with_s, base + sh, rtol=1e-12, atol=1e-15)


def _bf16_round(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_inputs_and_intermediate():
    rng = np.random.default_rng(3)
    x, w13, w2, ids, w = rand_problem(rng, T=16, H=64, I=32, E=3, K=2)
    xb = oracle.bf16_encode(x); w13b = oracle.bf16_encode(w13); w2b = oracle.bf16_encode(w2)
    out, _ = oracle.moe_layer(xb, w13b, w2b, ids, w, w_dtype="bf16", x_dtype="bf16", inter="bf16")
    xd, w13d, w2d = (oracle.bf16_decode(v) for v in (xb, w13b, w2b))
    # the decoded operands agree with torch's own bf16 casts
    assert np.array_equal(xd, torch.from_numpy(x).to(torch.bfloat16).double().numpy())
    ref = dense_layer(xd, w13d, w2d, ids, w, 3, round_a=_bf16_round)
    nr = dense_layer(xd, w13d, w2d, ids, w, 3)
    err = np.max(np.abs(out - ref)) / np.max(np.abs(ref))
    assert err < 1e-6
    # and the rounding hook is really on: without it the result moves by ~bf16 ulps
    assert np.max(np.abs(out - nr)) / np.max(np.abs(nr)) > 1e-5


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def test_token_quant_bound_and_library():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1, (64, 300)).astype(np.float32)
    x[3] = 0.0
    x[5, :] = 1e-3 * x[5, :]
    xb = oracle.bf16_encode(x)
    xd = oracle.bf16_decode(xb).astype(np.float32)
    q, s = oracle.quant_tokens_e4m3(xb)
    assert s[3] == 1.0 and np.all(q[3] == 0)
    dq = oracle.e4m3_decode(q) * s[:, None].astype(np.float64)
    amax = np.abs(xd).max(1)
    for t in range(64):
        if amax[t] == 0:
            continue
        assert s[t] == np.float32(amax[t] / np.float32(448.0))
        j = np.argmax(np.abs(xd[t]))
        assert q[t, j] in (0x7E, 0xFE)
        # half-ulp bound of E4M3: 2^-4 relative for normals, 2^-10 absolute below 2^-6
        bound = np.maximum(np.abs(xd[t]) * 2.0 ** -4, 2.0 ** -10 * s[t]) * (1 + 1e-6)
        assert np.all(np.abs(dq[t] - xd[t]) <= bound)
        inv = np.float32(448.0) / np.float32(amax[t])
        lib = _torch_e4m3(xd[t] * inv)
        assert np.array_equal(oracle.e4m3_decode(q[t]), lib)


def test_fp8_layer_against_dense_with_library_casts():
    rng = np.random.default_rng(5)
    T, H, I, E, K = 12, 64, 32, 3, 2
    x, w13, w2, ids, w = rand_problem(rng, T=T, H=H, I=I, E=E, K=K)
    xb = oracle.bf16_encode(x)
    # per-row weight quantisation with torch's cast (input preparation)
    def qrows(m):
        amax = np.abs(m).max(-1, keepdims=True).astype(np.float32)
        codes = torch.from_numpy((m * (np.float32(448) / amax)).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        return codes, (amax[..., 0] / np.float32(448)).astype(np.float32)
    w13q, s13 = qrows(w13)
    w2q, s2 = qrows(w2)
    out, _ = oracle.moe_layer(xb, w13q, w2q, ids, w, w_dtype="e4m3", x_dtype="bf16", inter="e4m3",
                              w13_scale=s13, w2_scale=s2)
    # dense formulation with torch casts for x and the intermediate
    xd = oracle.bf16_decode(xb).astype(np.float32)
    amax = np.abs(xd).max(1)
    sx = (amax / np.float32(448)).astype(np.float32)
    xq = np.stack([_torch_e4m3(xd[t] * (np.float32(448) / amax[t])) for t in range(T)]) * sx[:, None]
    w13d = oracle.e4m3_decode(w13q) * s13[..., None]
    w2d = oracle.e4m3_decode(w2q) * s2[..., None]

    def requant(a):
        a32 = a.astype(np.float32)
        am = np.abs(a32).max(1)
        sa = (am / np.float32(448)).astype(np.float64)
        return np.stack([_torch_e4m3(a32[t] * (np.float32(448) / am[t])) for t in range(len(a))]) \
            * sa[:, None]
    ref = dense_layer(xq, w13d, w2d, ids, w, E, round_a=requant)
    err = np.max(np.abs(out - ref)) / np.max(np.abs(ref))
    assert err < 1e-5, err
    # sanity: the fp8 layer approximates the unquantised fp64 layer (E4M3 keeps 3
    # mantissa bits, so a few per cent on short dot products)
    exact = dense_layer(xd.astype(np.float64), w13.astype(np.float64), w2.astype(np.float64),
                        ids, w, E)
    assert np.max(np.abs(out - exact)) / np.max(np.abs(exact)) < 0.15


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def mxfp4_random(rng, rows, cols):
    """Random MXFP4 operands and their exact float values, built independently
    of the oracle: nibbles, one E8M0 byte per 32 elements of a row, the even
    column in the low nibble."""
    nib = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    sc = rng.integers(120, 125, (rows, cols // 32)).astype(np.uint8)
    vals = E2M1[nib] * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc, vals


def test_mxfp4_layer_against_dense_with_float_weights():
    rng = np.random.default_rng(7)
    T, H, I, E, K = 10, 64, 96, 3, 2
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    parts13 = [mxfp4_random(rng, 2 * I, H) for _ in range(E)]
    parts2 = [mxfp4_random(rng, H, I) for _ in range(E)]
    w13q = np.stack([p[0] for p in parts13]); s13 = np.stack([p[1] for p in parts13])
    w2q = np.stack([p[0] for p in parts2]); s2 = np.stack([p[1] for p in parts2])
    w13d = np.stack([p[2] for p in parts13]); w2d = np.stack([p[2] for p in parts2])
    xb = oracle.bf16_encode(x)
    out, _ = oracle.moe_layer(xb, w13q, w2q, ids, w, w_dtype="e2m1", x_dtype="bf16", inter="e4m3",
                              w13_scale=s13, w2_scale=s2)
    xd = oracle.bf16_decode(xb).astype(np.float32)
    amax = np.abs(xd).max(1)
    sx = (amax / np.float32(448)).astype(np.float32)
    xq = np.stack([_torch_e4m3(xd[t] * (np.float32(448) / amax[t])) for t in range(T)]) * sx[:, None]

    def requant(a):
        a32 = a.astype(np.float32)
        am = np.abs(a32).max(1)
        sa = (am / np.float32(448)).astype(np.float64)
        return np.stack([_torch_e4m3(a32[t] * (np.float32(448) / am[t])) for t in range(len(a))]) \
            * sa[:, None]
    ref = dense_layer(xq, w13d, w2d, ids, w, E, round_a=requant)
    err = np.max(np.abs(out - ref)) / np.max(np.abs(ref))
    assert err < 1e-5, err
    # a wrong nibble order or block index would change the values: swap the
    # nibbles of one expert's gate rows and the result must move
    w13s = w13q.copy()
    w13s[0] = (w13s[0] >> 4) | ((w13s[0] & 15) << 4)
    out_s, _ = oracle.moe_layer(xb, w13s, w2q, ids, w, w_dtype="e2m1", x_dtype="bf16", inter="e4m3",
                                w13_scale=s13, w2_scale=s2)
    assert np.max(np.abs(out_s - out)) > 1e-3 * np.max(np.abs(out))
