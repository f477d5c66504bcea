"""The seeded generators: the tensor hash equals its pure-Python definition,
the distributions have the stated moments and bounds, Zipf ids are distinct
per token and follow the law, and slabs regenerate identically."""
import numpy as np
import torch

import moe_synth as ms


def test_tensor_hash_matches_python_definition():
    for (seed, tag, block, stream) in ((0, 1, 0, 0), (7, 3, 5, 1), (0, 2, 255, 0)):
        starts = [0, 12345, (1 << 32) - 64]
        for s0 in starts:
            h = ms.hash_u32(seed, tag, block, s0, 64, stream=stream).tolist()
            assert h == [ms.hash_u32_reference(seed, tag, block, s0 + i, stream) for i in range(64)]


def test_normal_and_uniform_moments():
    z = ms.normal(0, 1, (1 << 20,), 1.0).double()
    assert abs(z.mean().item()) < 5e-3 and abs(z.std().item() - 1) < 5e-3
    assert z.abs().max().item() <= 2 * 3 ** 0.5
    z2 = ms.normal(0, 1, (1 << 16,), 0.02).double()
    assert abs(z2.std().item() - 0.02) < 5e-4
    u = ms.uniform(0, 5, (1 << 18,), -0.1, 0.1).double()
    assert u.min().item() >= -0.1 and u.max().item() < 0.1 and abs(u.mean().item()) < 1e-3


def test_slab_regeneration_is_bit_identical():
    cfg = ms.scaled("decode_bf16", H=64, I=32, E=6)
    full = ms.make_weights(cfg)
    part = ms.make_weights(cfg, experts=[4, 1])
    assert torch.equal(full["w13"][4].view(torch.int16), part["w13"][0].view(torch.int16))
    assert torch.equal(full["w2"][1].view(torch.int16), part["w2"][1].view(torch.int16))


def test_zipf_ids():
    ids = ms.zipf_topk_ids(0, ms.TAG_IDS, 20000, 8, 256, 1.1)
    assert ids.shape == (20000, 8) and ids.min() >= 0 and ids.max() < 256
    srt = np.sort(ids, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0)                 # no repeats within a token
    cnt = np.sort(np.bincount(ids.ravel(), minlength=256))[::-1]
    assert cnt[0] > 5 * cnt[50] > 0                          # heavy head
    one = ms.zipf_topk_ids(0, ms.TAG_IDS, 50000, 1, 32, 1.2)[:, 0]
    c = np.sort(np.bincount(one, minlength=32))[::-1].astype(np.float64)
    p = np.arange(1, 33) ** -1.2
    assert np.allclose(c / c.sum(), p / p.sum(), atol=0.01)


def test_uniform_assignment_is_exact():
    cfg = ms.CONFIGS["prefill_bf16"]
    a = ms.assigned_experts(cfg)
    assert np.all(np.bincount(a, minlength=32) == 64)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mx_decode(packed, sc):
    nib = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], -1)
    mag = E2M1_GRID[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return mag * np.ldexp(1.0, np.repeat(sc.astype(np.int64) - 127, 32, axis=1))


def test_mxfp4_input_preparation():
    w = ms.normal_slab(0, ms.TAG_W13, 3, (40, 256), 0.02, "cpu")
    w[5, 32:64] = 0.0                                           # an all-zero block
    q, sc = ms.quantise_rows_mxfp4_input(w)
    assert q.shape == (40, 128) and sc.shape == (40, 8)
    q, sc, wd = q.numpy(), sc.numpy(), w.double().numpy()
    scale = np.ldexp(1.0, sc.astype(np.int64) - 127)
    amax = np.abs(wd).reshape(40, 8, 32).max(-1)
    nz = amax > 0
    ratio = amax[nz] / scale[nz]
    assert ratio.min() >= 4.0 and ratio.max() < 8.0            # exponent = floor(log2 amax) - 2
    assert sc[5, 1] == 127 and not q[5, 16:32].any()
    dec = _mx_decode(q, sc)
    v = wd / np.repeat(scale, 32, axis=1)
    inside = np.abs(v) <= 6.0
    step = np.where(np.abs(v) < 2.0, 0.5, np.where(np.abs(v) < 4.0, 1.0, 2.0))
    err = np.abs(dec / np.repeat(scale, 32, axis=1) - v)
    assert (err[inside] <= step[inside] / 2).all()
    assert np.array_equal(dec[~inside] / np.repeat(scale, 32, axis=1)[~inside], 6.0 * np.sign(v[~inside]))


def test_mxfp4_midpoints_round_to_even_codes_and_pack_low_nibble_first():
    # one block whose amax is 6 (exponent 0): the midpoints between grid values
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]                                 # even code on a tie
    row = torch.zeros(1, 32)
    row[0, :7] = torch.tensor(mids)
    row[0, 7] = 6.0
    row[0, 8] = -1.0
    q, sc = ms.quantise_rows_mxfp4_input(row)
    assert sc[0, 0].item() == 127
    nib = np.stack([q.numpy() & 15, q.numpy() >> 4], axis=-1).reshape(-1)
    assert list(nib[:7]) == want
    assert nib[7] == 7 and nib[8] == (8 | 2)                     # 6.0 and -1.0
    assert (q.numpy()[0, 0] & 15) == nib[0] and (q.numpy()[0, 0] >> 4) == nib[1]
