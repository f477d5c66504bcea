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
