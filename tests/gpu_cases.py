"""Shared helpers for the GPU parity tests: cached synthetic inputs (host
and device), the layer run through the C ABI, and tolerance helpers."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import synth
import sparse_mixture_experts_softmax_amd as moe

CONFIG_NAMES = ["tiny", "decode", "medium", "prefill", "skewed", "large"]


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def _weights(E, H, I, seed):
    shape = synth.MoEShape("w", 1, H, E, 1, I)
    return synth.expert_weights(shape, seed)


@functools.lru_cache(maxsize=8)
def host_inputs(name: str, seed: int = 0, T: int = -1):
    shape = synth.CONFIGS[name]
    if T >= 0:
        shape = shape.with_tokens(T)
    inp = synth.make_inputs(shape, seed=seed, weights=False)
    inp.w13, inp.w2 = _weights(shape.E, shape.H, shape.I, seed)
    return inp


def custom_inputs(name, T, H, E, k, I, norm=True, skewed=False, seed=0):
    shape = synth.MoEShape(name, T, H, E, k, I, norm_topk_prob=norm, skewed=skewed)
    return synth.make_inputs(shape, seed=seed)


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


_device_cache = {}


def device_inputs(inp, key=None):
    """Device copies of an input set (cached by key; weights shared by key)."""
    if key is not None and key in _device_cache:
        return _device_cache[key]
    d = dict(
        x=bf16_tensor(inp.x),
        w_router=bf16_tensor(inp.w_router),
        w13=bf16_tensor(inp.w13),
        w2=bf16_tensor(inp.w2),
        bias=None if inp.router_bias is None else torch.from_numpy(inp.router_bias).cuda(),
    )
    d["packed"] = moe.pack_experts(d["w13"], d["w2"])
    if key is not None:
        _device_cache.clear()  # keep one full-size set resident at a time
        _device_cache[key] = d
    return d


def run_layer(inp, dev=None, block_m=None, out_dtype=torch.bfloat16, y_dtype=torch.float16):
    """The layer through the C ABI; returns (out, buffers)."""
    s = inp.shape
    dev = dev or device_inputs(inp)
    bufs = moe.allocate(s.T, s.H, s.E, s.k, s.I, "cuda", block_m, out_dtype, y_dtype)
    out = moe.moe_layer(dev["x"], dev["w_router"], top_k=s.k, packed=dev["packed"],
                        norm_topk_prob=s.norm_topk_prob, router_bias=dev["bias"], buffers=bufs)
    torch.cuda.synchronize()
    return out, bufs


def pack_reference(w: np.ndarray, gated: bool) -> np.ndarray:
    """The packed fragment layout built with numpy from its definition:
    16-row bands x 32-column k-steps, block = 64 lanes x 8 values, lane l
    holding row l%16 at columns 8*(l//16)..; gate/up bands interleaved."""
    E, N, K = w.shape
    if gated:
        I = N // 2
        g = w[:, :I].reshape(E, I // 16, 16, K)
        u = w[:, I:].reshape(E, I // 16, 16, K)
        bands = np.stack([g, u], axis=2).reshape(E, N // 16, 16, K)
    else:
        bands = w.reshape(E, N // 16, 16, K)
    b = bands.reshape(E, N // 16, 16, K // 32, 4, 8)  # e, band, row, kstep, chunk, 8
    return np.ascontiguousarray(b.transpose(0, 1, 3, 4, 2, 5)).reshape(E, N, K)


def act_rows(act: torch.Tensor) -> torch.Tensor:
    """Row-major [cap, I] view of act, which the GEMMs store as fragment
    blocks (16 rows x 32 columns per block, lane l holding row l%16 at
    columns 8*(l//16)..; the layout of the packed weights)."""
    cap, I = act.shape
    return act.reshape(cap // 16, I // 32, 4, 16, 8).permute(0, 3, 1, 2, 4).reshape(cap, I)


def act_blocks(rows: torch.Tensor) -> torch.Tensor:
    """Inverse of act_rows: row-major rows to the fragment-block layout."""
    cap, I = rows.shape
    return rows.reshape(cap // 16, 16, I // 32, 4, 8).permute(0, 2, 3, 1, 4).reshape(cap, I).contiguous()


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and ragged-tail tokens plus a seeded random sample."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    fixed = {0, 1, T - 1, T - 2, (T // 16) * 16 - 1, T // 2}
    rest = rng.choice(T, size=n, replace=False)
    return np.array(sorted(fixed | set(rest.tolist())))[: max(n, len(fixed))]


def layer_tolerance(ref: np.ndarray, floor: bool = True) -> float:
    """max |err| bound for the layer output: 2e-2 * rms(out) + 1e-3."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return 2e-2 * rms + (1e-3 if floor else 0.0)


def logits_bound(inp, tokens=None) -> np.ndarray:
    """Per-logit bound on fp32 accumulation of H exact bf16 products (any
    summation order): H * 2^-24 * sum_h |x_h w_eh| + 2^-24 |bias_e|."""
    x = synth.bf16_to_f64(inp.x if tokens is None else inp.x[tokens])
    wr = synth.bf16_to_f64(inp.w_router)
    H = x.shape[1]
    b = 0.0 if inp.router_bias is None else np.abs(inp.router_bias.astype(np.float64))
    return (H + 1) * 2.0 ** -24 * (np.abs(x) @ np.abs(wr).T + b)
