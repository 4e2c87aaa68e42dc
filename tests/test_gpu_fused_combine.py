"""The weighted combine fused into the down projection
(moe_grouped_gemm_down_combine) against the two separate calls it replaces
(moe_grouped_gemm_down, then moe_combine) and against the oracle.

The fused kernel sums a token's k rows in slot order with the same fp32
arithmetic as moe_combine, whichever workgroup finishes the token: the
outputs must be the same bits as the separate path, on every workload, row
tile size and output precision, call after call (the arrival counters must
come back to zero)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_softmax_amd as moe
from gpu_cases import (CONFIG_NAMES, bf16_tensor, custom_inputs, device_inputs, host_inputs, layer_tolerance, log,
                       to_bits)

pytestmark = pytest.mark.gpu
F16, F32, BF16 = torch.float16, torch.float32, torch.bfloat16


def _run(inp, dev, block_m=None, y_dtype=F16, out_dtype=BF16):
    """(fused out, separate out, fused buffers) on the same routing."""
    s = inp.shape
    b = moe.allocate(s.T, s.H, s.E, s.k, s.I, "cuda", block_m, out_dtype, y_dtype)
    sep = moe.moe_layer(dev["x"], dev["w_router"], top_k=s.k, packed=dev["packed"], norm_topk_prob=s.norm_topk_prob,
                        router_bias=dev["bias"], buffers=b).clone()
    y_sep = b.y.clone()
    b.y.fill_(float("nan"))
    b.out.fill_(float("nan"))
    fused = moe.moe_layer(dev["x"], dev["w_router"], top_k=s.k, packed=dev["packed"],
                          norm_topk_prob=s.norm_topk_prob, router_bias=dev["bias"], buffers=b, fused_combine=True)
    torch.cuda.synchronize()
    assert torch.equal(b.y, y_sep), "y differs between the fused and the separate down projection"
    return fused, sep, b


@pytest.mark.parametrize("name", CONFIG_NAMES)
@pytest.mark.parametrize("y_dtype,out_dtype", [(F16, BF16), (F32, F32)])
def test_fused_combine_same_bits_as_separate(name, y_dtype, out_dtype):
    log(f"fused combine {name} y {y_dtype} out {out_dtype}")
    inp = host_inputs(name)
    dev = device_inputs(inp, key=name)
    fused, sep, b = _run(inp, dev, y_dtype=y_dtype, out_dtype=out_dtype)
    assert torch.equal(fused, sep)
    assert not b.counters.any(), "arrival counters not reset"
    # a second call on the same buffers (counters reused) gives the same bits
    s = inp.shape
    again = moe.moe_layer(dev["x"], dev["w_router"], top_k=s.k, packed=dev["packed"],
                          norm_topk_prob=s.norm_topk_prob, router_bias=dev["bias"], buffers=b, fused_combine=True)
    torch.cuda.synchronize()
    assert torch.equal(again, sep)
    assert not b.counters.any()


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,H,E,k,I", [(700, 192, 8, 2, 160), (333, 320, 16, 4, 96), (45, 128, 1, 1, 64),
                                       (20, 64, 8, 8, 32)])
def test_fused_combine_tile_sizes_and_ragged_groups(bm, T, H, E, k, I):
    """H not a multiple of the 128-column group (192, 320, 64), I with a
    ragged last k-step, k = E, one expert, every row tile size."""
    inp = custom_inputs(f"fc{T}_{H}", T, H, E, k, I, seed=T + H)
    dev = device_inputs(inp)
    fused, sep, b = _run(inp, dev, block_m=bm)
    assert torch.equal(fused, sep)
    assert not b.counters.any()


def test_fused_combine_against_oracle_every_token():
    inp = host_inputs("prefill")
    s = inp.shape
    dev = device_inputs(inp, key="prefill")
    b = moe.allocate(s.T, s.H, s.E, s.k, s.I, "cuda", None, F32, F32)
    out = moe.moe_layer(dev["x"], dev["w_router"], top_k=s.k, packed=dev["packed"], norm_topk_prob=s.norm_topk_prob,
                        buffers=b, fused_combine=True)
    torch.cuda.synchronize()
    ref, _, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    log(f"  prefill fused: max err {err:.3e}, bound {layer_tolerance(ref):.3e}")
    assert err <= layer_tolerance(ref)


def test_fused_combine_fp32_y_beyond_fp16_range():
    """With fp32 y the fused path has no fp16 range limit: down weights scaled
    by 2^23 still match the oracle."""
    base = custom_inputs("fcbig", 160, 256, 8, 2, 128, seed=21)
    w2 = (synth.bf16_to_f64(base.w2) * 2.0 ** 23).astype(np.float32)
    w2_bits = (w2.view(np.uint32) >> 16).astype(np.uint16)
    inp = synth.MoEInputs(base.shape, base.seed, base.x, base.w_router, base.w13, w2_bits, None)
    dev = device_inputs(inp)
    for bm in (16, 32, 128):
        fused, sep, b = _run(inp, dev, block_m=bm, y_dtype=F32, out_dtype=F32)
        assert torch.equal(fused, sep)
        ref, _, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 2, True)
        got = fused.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all() and np.abs(ref).max() > 1e5
        assert np.abs(got - ref).max() <= layer_tolerance(ref)
