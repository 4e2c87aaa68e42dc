"""Dense SwiGLU GatedMLP through the grouped GEMMs (one expert, every token
routed to it with weight 1) against the oracle's expert MLP."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_softmax_amd as moe
from gpu_cases import bf16_tensor, layer_tolerance, log, sample_tokens, to_bits

pytestmark = pytest.mark.gpu


def _dense_inputs(T, H, I, seed):
    shape = synth.MoEShape("dense", T, H, 1, 1, I)
    w13, w2 = synth.expert_weights(shape, seed)
    x = synth.normal_bf16(seed, synth.TAG_X, (T, H), 1.0)
    return x, w13, w2


@pytest.mark.parametrize("T,H,I,bm", [(4096, 1024, 3072, None), (1000, 1024, 3072, 128), (37, 256, 96, 32),
                                      (1, 512, 64, 16), (300, 2048, 768, 64)])
def test_dense_mlp_matches_oracle(T, H, I, bm):
    log(f"dense T={T} H={H} I={I} block_m={bm}")
    x, w13, w2 = _dense_inputs(T, H, I, seed=T)
    packed = moe.pack_experts(bf16_tensor(w13), bf16_tensor(w2))
    out = moe.gated_mlp(bf16_tensor(x), packed, block_m=bm)
    torch.cuda.synchronize()
    rows = sample_tokens(T, 64)
    ref = oracle.expert_mlp(synth.bf16_to_f64(x[rows]), w13[0], w2[0])
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    err = np.abs(got - ref).max()
    log(f"  max err {err:.3e} bound {layer_tolerance(ref):.3e}")
    assert np.isfinite(got).all()
    assert err <= layer_tolerance(ref)
    # elementwise: the output's bf16 rounding (<= 2^-9 |out|) plus the bf16
    # rounding of act carried through the down projection (random, standard
    # deviation about 2^-9/sqrt(3) rms(out) ~ 1.1e-3 rms(out); 8e-3 rms(out)
    # covers the tails of ~65k samples)
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 8e-3 * np.sqrt(np.mean(ref ** 2))).all()


def test_dense_mlp_equals_moe_layer_with_one_expert():
    T, H, I = 513, 512, 256
    x, w13, w2 = _dense_inputs(T, H, I, seed=3)
    packed = moe.pack_experts(bf16_tensor(w13), bf16_tensor(w2))
    wr = bf16_tensor(synth.normal_bf16(3, synth.TAG_WR, (1, H), 0.02))
    for bm in (16, 128):
        a = moe.gated_mlp(bf16_tensor(x), packed, block_m=bm)
        b = moe.moe_layer(bf16_tensor(x), wr, top_k=1, packed=packed, block_m=bm)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(a), to_bits(b))


@pytest.mark.parametrize("T,H,I", [(1000, 1024, 3072), (4096, 1024, 3072), (129, 512, 256)])
def test_dense_finer_down_blocks_same_bits(T, H, I):
    """With the block size left to the library the down projection of a
    narrow layer runs on 64-row blocks (its own grouping, the identity
    again) while gate/up keeps 128-row blocks: the same MFMA shape and k
    order per element, so the output equals the all-128-row run bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert moe.dense_down_block_m(T, H, moe.moe_pick_block_m(T, 1, 1), cus) == 64
    x, w13, w2 = _dense_inputs(T, H, I, seed=T + 1)
    packed = moe.pack_experts(bf16_tensor(w13), bf16_tensor(w2))
    auto = moe.gated_mlp(bf16_tensor(x), packed)
    fixed = moe.gated_mlp(bf16_tensor(x), packed, block_m=128)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(auto), to_bits(fixed))
