"""The fragment-block layout of act, as the GPU tests unpack it, against the
layout definition of the packed weights (built with numpy from that
definition), on the CPU."""
import numpy as np
import torch

from gpu_cases import act_blocks, act_rows, pack_reference


def test_act_blocks_is_the_packed_weight_layout():
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 1 << 16, size=(48, 96), dtype=np.uint16)
    t = torch.from_numpy(rows.view(np.int16))
    got = act_blocks(t).numpy().view(np.uint16)
    assert np.array_equal(got, pack_reference(rows[None], gated=False)[0])
    assert np.array_equal(act_rows(act_blocks(t)).numpy(), t.numpy())


def test_fragment_index_formula():
    """Element (r, c) sits at ((r//16)*(I//32) + c//32)*512 + (16*((c%32)//8) + r%16)*8 + c%8."""
    cap, I = 32, 64
    rows = torch.arange(cap * I, dtype=torch.int32).reshape(cap, I)
    flat = act_blocks(rows).reshape(-1)
    for r in range(cap):
        for c in range(0, I, 5):
            idx = ((r // 16) * (I // 32) + c // 32) * 512 + (16 * ((c % 32) // 8) + r % 16) * 8 + c % 8
            assert int(flat[idx]) == r * I + c
