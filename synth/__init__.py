"""Seeded synthetic inputs for the sparse MoE layer.

This module is shared by the CPU oracle's tests and by the HIP path's tests
and bench. It draws inputs only; it computes none of the layer's outputs.
The one place it touches the router product is the top-k margin screen: it
evaluates the token-by-expert logits in float64 with a numpy matmul purely to
reject and redraw activation rows whose k+1 largest logits are closer than
``MARGIN``, so that fp32 (GPU) and fp64 (oracle) logits select the same
experts. Nothing it computes is used as an expected value.

Shapes and distributions follow the five workloads the layer is specified on
(tiny, decode, prefill, skewed routing, large): activations N(0,1) and all
weights N(0,0.02), rounded to bfloat16 with round-to-nearest-even. The expert
weight layout is the packed one from the model-and-weights page of the
handbook ("stream weight loading": per-expert tensors stacked into one
[E, ...] tensor): ``w13`` is [E, 2I, H] with gate rows first, then up rows
(merged gate_up projection), ``w2`` is [E, H, I].
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
# MOE_SYNTH_LIB names another build (the host-sanitizer test build).
_LIB_PATH = os.environ.get("MOE_SYNTH_LIB") or os.path.join(_HERE, "libmoe_synth.so")
_lib = None

MARGIN = 1e-3  # minimum adjacent gap among each token's k+1 largest fp64 logits
MAX_REDRAWS = 64

# Stream tags (any distinct 64-bit values).
TAG_X = 0x100  # activation row redraw a uses TAG_X + a
TAG_WR = 0x2
TAG_W13 = 0x3
TAG_W2 = 0x4
TAG_RANK = 0x5

# Skewed-routing recipe: experts get a seeded popularity rank r (1 = most
# popular). The NUM_EMPTY least popular receive a bias that removes them from
# every top-k; the others get bias -ZIPF_S * SKEW_C * ln(r). With SKEW_C = 0.5
# the realised loads at the skewed workload fall on a log-log line of slope
# about -1.2 (checked by a test against the oracle's routing).
ZIPF_S = 1.2
SKEW_C = 0.5
NUM_EMPTY = 10
EMPTY_BIAS = -30.0


def build(force: bool = False) -> str:
    """Compile the generator with gcc (OpenMP) into this directory."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ctypes.c_double, p]
        lib.synth_normal_f64.argtypes = [u64, u64, u64, u64, ctypes.c_double, p]
        lib.synth_u64.argtypes = [u64, u64, u64, u64, p]
        for f in (lib.synth_normal_bf16, lib.synth_normal_f64, lib.synth_u64):
            f.restype = None
        _lib = lib
    return _lib


def normal_bf16(seed: int, tag: int, shape, std: float, start: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of std*N(0,1), elements start.. of stream (seed, tag)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, tag, start, n, std, out.ctypes.data)
    return out.reshape(shape)


def normal_f64(seed: int, tag: int, n: int, std: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_normal_f64(seed, tag, start, n, std, out.ctypes.data)
    return out


def u64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        _load().synth_u64(seed, tag, start, n, out.ctypes.data)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """Field names follow the MoE fields of the model config (hidden_size,
    num_experts, num_experts_per_tok, moe_intermediate_size, norm_topk_prob)."""

    name: str
    num_tokens: int
    hidden_size: int
    num_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    norm_topk_prob: bool = True
    skewed: bool = False

    @property
    def T(self):
        return self.num_tokens

    @property
    def H(self):
        return self.hidden_size

    @property
    def E(self):
        return self.num_experts

    @property
    def k(self):
        return self.num_experts_per_tok

    @property
    def I(self):  # noqa: E743
        return self.moe_intermediate_size

    def with_tokens(self, T: int) -> "MoEShape":
        return dataclasses.replace(self, num_tokens=T)


CONFIGS = {
    "tiny": MoEShape("tiny", 16, 64, 8, 2, 32),
    "decode": MoEShape("decode", 64, 2048, 128, 8, 768),
    "prefill": MoEShape("prefill", 4096, 2048, 128, 8, 768),
    "skewed": MoEShape("skewed", 16384, 2048, 128, 8, 768, skewed=True),
    "large": MoEShape("large", 8192, 4096, 128, 8, 1536),
    # Between the decode- and prefill-shaped layers of the same model: 512
    # tokens, 32 (token, slot) rows per expert on average.
    "medium": MoEShape("medium", 512, 2048, 128, 8, 768),
    # Dense SwiGLU MLP of the Qwen3-0.6B layer the op-layer page prints
    # (gate_up_proj (6144, 1024), down_proj (1024, 3072)): one expert, k = 1.
    "dense": MoEShape("dense", 4096, 1024, 1, 1, 3072),
}


@dataclasses.dataclass
class MoEInputs:
    """Host-side inputs. bf16 tensors are uint16 bit patterns."""

    shape: MoEShape
    seed: int
    x: np.ndarray  # [T, H]
    w_router: np.ndarray  # [E, H]
    w13: Optional[np.ndarray]  # [E, 2I, H] (None when weights are generated lazily)
    w2: Optional[np.ndarray]  # [E, H, I]
    router_bias: Optional[np.ndarray]  # [E] float32 or None
    redraws: int = 0  # activation rows redrawn by the margin screen


def skew_bias(seed: int, E: int) -> np.ndarray:
    """Per-expert logit bias for the skewed-routing workload (float32)."""
    order = np.argsort(u64(seed, TAG_RANK, E), kind="stable")  # seeded permutation
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    bias = -ZIPF_S * SKEW_C * np.log(rank.astype(np.float64))
    bias[rank > E - NUM_EMPTY] = EMPTY_BIAS
    return bias.astype(np.float32)


def _margin_violations(x64: np.ndarray, wr64: np.ndarray, bias: Optional[np.ndarray], k: int) -> np.ndarray:
    lg = x64 @ wr64.T
    if bias is not None:
        lg = lg + bias.astype(np.float64)[None, :]
    E = lg.shape[1]
    m = min(k + 1, E)
    top = -np.sort(-lg, axis=1)[:, :m]
    if m < 2:
        return np.zeros(lg.shape[0], dtype=bool)
    gaps = top[:, :-1] - top[:, 1:]
    return (gaps < MARGIN).any(axis=1)


def make_inputs(shape: MoEShape, seed: int = 0, weights: bool = True, margin: bool = True) -> MoEInputs:
    """Generate one workload's inputs. ``weights=False`` skips w13/w2 (they can
    be produced later by :func:`expert_weights`)."""
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I
    wr = normal_bf16(seed, TAG_WR, (E, H), 0.02)
    bias = skew_bias(seed, E) if shape.skewed else None
    x = normal_bf16(seed, TAG_X, (T, H), 1.0)
    redraws = 0
    if margin and T > 0:
        wr64 = bf16_to_f64(wr)
        bad = np.nonzero(_margin_violations(bf16_to_f64(x), wr64, bias, k))[0]
        attempt = 0
        while bad.size:
            attempt += 1
            if attempt > MAX_REDRAWS:
                raise RuntimeError(f"margin screen did not converge for {bad.size} rows")
            for t in bad:
                x[t] = normal_bf16(seed, TAG_X + attempt, (H,), 1.0, start=int(t) * H)
            redraws += bad.size
            still = _margin_violations(bf16_to_f64(x[bad]), wr64, bias, k)
            bad = bad[still]
    w13 = w2 = None
    if weights:
        w13, w2 = expert_weights(shape, seed)
    return MoEInputs(shape, seed, x, wr, w13, w2, bias, redraws)


def expert_weights(shape: MoEShape, seed: int = 0, experts=None):
    """Packed expert weights (w13 [E,2I,H], w2 [E,H,I]) as bf16 bits; with
    ``experts`` given, only those experts' slices (same values as the full
    tensors)."""
    E, H, I = shape.E, shape.H, shape.I
    if experts is None:
        return (normal_bf16(seed, TAG_W13, (E, 2 * I, H), 0.02), normal_bf16(seed, TAG_W2, (E, H, I), 0.02))
    n13, n2 = 2 * I * H, H * I
    w13 = np.stack([normal_bf16(seed, TAG_W13, (2 * I, H), 0.02, start=int(e) * n13) for e in experts])
    w2 = np.stack([normal_bf16(seed, TAG_W2, (H, I), 0.02, start=int(e) * n2) for e in experts])
    return w13, w2
