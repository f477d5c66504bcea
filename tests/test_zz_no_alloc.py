"""The no-allocation Align & Sort (moe_align_sort_noalloc) through the C ABI:
the same bits as moe_align_sort with a caller workspace, on two calls in a
row (the second with a smaller input, so stale scratch contents from the
first call are there to trip over), on the one-workgroup path, and after a
call that the size limit rejects."""
import numpy as np
import pytest
import torch

import routing_align_sort_amd as moe
from gpu_helpers import device, say

pytestmark = pytest.mark.gpu


def zipf_ids(rng, T, K, E, s=1.1):
    """Ids of K distinct experts per token, Zipf(s) over E ranks (input
    shape and law of the align-only workload; drawn here with numpy)."""
    p = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    perm = rng.permutation(E)
    ids = np.empty((T, K), np.int32)
    for t in range(T):
        ids[t] = perm[rng.choice(E, size=K, replace=False, p=p)]
    return ids


def outputs(T, K, E, B, dev, fill):
    C = moe.moe_align_sort_capacity(T, K, E, B)
    return dict(sorted_token_ids=torch.full((C,), fill, dtype=torch.int32, device=dev),
                expert_ids=torch.full((C // B,), fill, dtype=torch.int32, device=dev),
                num_tokens_post_padded=torch.full((1,), fill, dtype=torch.int32, device=dev),
                expert_offsets=torch.full((E + 1,), fill, dtype=torch.int32, device=dev))


def check_same(ids_np, E, B, dev, label):
    T, K = ids_np.shape
    ids = torch.tensor(ids_np, device=dev)
    ref = moe.moe_align_sort(ids, E, B, **outputs(T, K, E, B, dev, -7))
    got = moe.moe_align_sort_noalloc(ids, E, B, **outputs(T, K, E, B, dev, 12345))
    torch.cuda.synchronize()
    for k in ("sorted_token_ids", "expert_ids", "num_tokens_post_padded", "expert_offsets"):
        assert torch.equal(got[k], ref[k]), (label, k)
    say(f"{label}: T={T} K={K} E={E} B={B}, P={int(ref['num_tokens_post_padded'].item())}: "
        f"no-alloc call equals the workspace call bit for bit")


def test_no_alloc_align_sort_equals_workspace_call():
    dev = device()
    rng = np.random.default_rng(11)
    limit = moe.moe_align_sort_noalloc_scratch_bytes()
    assert limit == 1088 * 1024
    # first call: the align-only workload's shape (16384 tokens x top-8 of 256, B 64)
    big = zipf_ids(rng, 16384, 8, 256)
    assert moe.moe_align_sort_workspace_bytes(16384, 8, 256, 64) <= limit
    check_same(big, 256, 64, dev, "call 1")
    # second call, smaller, with some ids out of range: the scratch keeps the
    # first call's counts, which must not leak into this result
    small = zipf_ids(rng, 3000, 4, 40)
    small[rng.random(small.shape) < 0.05] = -1
    check_same(small, 40, 16, dev, "call 2")
    # the one-workgroup path (no scratch used) and the many-workgroup path again
    check_same(zipf_ids(rng, 100, 8, 64), 64, 32, dev, "call 3")
    check_same(zipf_ids(rng, 9000, 8, 256), 256, 128, dev, "call 4")


def test_no_alloc_align_sort_rejects_inputs_beyond_the_scratch():
    dev = device()
    T, K, E, B = 1 << 20, 8, 1024, 16
    assert moe.moe_align_sort_workspace_bytes(T, K, E, B) > moe.moe_align_sort_noalloc_scratch_bytes()
    ids = torch.zeros((T, K), dtype=torch.int32, device=dev)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_align_sort_noalloc(ids, E, B, **outputs(T, K, E, B, dev, 0))
    assert ei.value.status == moe.MOE_ERR_SCRATCH_LIMIT
    # the library still works on the same device after the rejection
    rng = np.random.default_rng(3)
    check_same(zipf_ids(rng, 2000, 8, 256), 256, 64, dev, "after a rejected call")
