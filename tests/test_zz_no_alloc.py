"""The allocation-free grouping entry point (moe_align_by_expert_noalloc,
static device scratch) against moe_align_by_expert with a caller workspace:
bit-identical outputs on two calls in a row, the second with a smaller
input (the scratch keeps the first call's histograms), through the C ABI."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_softmax_amd as moe

pytestmark = pytest.mark.gpu


def _ids(T, k, E, seed):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    return torch.from_numpy(ids).cuda()


def _outputs(T, k, E, bm):
    cap = moe.moe_align_capacity(T, k, E, bm)
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((cap,), -9, **i32), torch.full((cap // bm,), -9, **i32), torch.full((E,), -9, **i32),
            torch.full((1,), -9, **i32))


def _with_workspace(ids, T, k, E, bm):
    out = _outputs(T, k, E, bm)
    wsb = moe.moe_align_workspace_bytes(T, k, E, bm)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda") if wsb else None
    moe.moe_align_by_expert(ids, T, k, E, bm, *out, ws)
    return out


def _noalloc(ids, T, k, E, bm):
    out = _outputs(T, k, E, bm)
    moe.moe_align_by_expert_noalloc(ids, T, k, E, bm, *out)
    return out


@pytest.mark.parametrize("first,second", [
    ((16384, 8, 128, 128, 1), (4096, 8, 128, 64, 2)),   # 32 tiles, then 32 smaller tiles
    ((20000, 8, 200, 32, 3), (3000, 4, 200, 16, 4)),    # 40 tiles of 4096 pairs, then 12
    ((65536, 8, 128, 128, 5), (900, 8, 128, 16, 6)),    # 128 tiles, then a single tile (no scratch)
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for T, k, E, bm, seed in (first, second):
        print(f"noalloc T={T} k={k} E={E} block_m={bm}", flush=True)
        assert moe.moe_align_workspace_bytes(T, k, E, bm) <= moe.moe_align_noalloc_max_workspace_bytes()
        ids = _ids(T, k, E, seed)
        ref = _with_workspace(ids, T, k, E, bm)
        got = _noalloc(ids, T, k, E, bm)
        torch.cuda.synchronize()
        for r, g, name in zip(ref, got, ("sorted_ids", "block_expert", "expert_counts", "num_padded")):
            assert torch.equal(r, g), f"{name} differs for T={T} k={k} E={E} block_m={bm}"


def test_noalloc_rejects_sizes_beyond_its_scratch():
    T, k, E, bm = 300000, 8, 256, 128  # 586 tiles x 256 experts of counts > 256 KB
    assert moe.moe_align_workspace_bytes(T, k, E, bm) > moe.moe_align_noalloc_max_workspace_bytes()
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    out = _outputs(T, k, E, bm)
    with pytest.raises(moe.MoEError, match="static scratch"):
        moe.moe_align_by_expert_noalloc(ids, T, k, E, bm, *out)
    torch.cuda.synchronize()
    assert (out[3] == -9).all()  # nothing was enqueued
