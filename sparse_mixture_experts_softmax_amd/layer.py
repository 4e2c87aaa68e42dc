"""The whole sparse MoE layer: allocates the intermediates with torch and
calls the five library entry points in order on one stream.

MoEConfig keeps the MoE field names of the model configuration on the
"Models and weight loading" page (hidden_size, num_experts,
num_experts_per_tok, moe_intermediate_size, norm_topk_prob, hidden_act);
like that page's GatedMLP, only the silu activation is accepted.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    hidden_size: int
    num_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    norm_topk_prob: bool = False
    hidden_act: str = "silu"

    def __post_init__(self):
        if self.hidden_act != "silu":
            raise ValueError(f"Unsupported activation: {self.hidden_act}")


@dataclasses.dataclass
class PackedExperts:
    """Expert weights in the grouped GEMMs' fragment layout (moe_pack_weights)."""

    w13: torch.Tensor  # packed [E, 2I, H]
    w2: torch.Tensor  # packed [E, H, I]
    num_experts: int
    hidden_size: int
    intermediate_size: int


def pack_experts(w13: torch.Tensor, w2: torch.Tensor, stream=None) -> PackedExperts:
    """Pack row-major w13 [E, 2I, H] (gate rows, then up rows) and w2 [E, H, I]
    once, at load time."""
    E, two_i, H = w13.shape
    I = two_i // 2
    if tuple(w2.shape) != (E, H, I):
        raise ValueError(f"w2 must be [E, H, I] = {(E, H, I)}, got {tuple(w2.shape)}")
    p13 = torch.empty_like(w13)
    p2 = torch.empty_like(w2)
    _lib.moe_pack_weights(w13, p13, E, 2 * I, H, True, stream)
    _lib.moe_pack_weights(w2, p2, E, H, I, False, stream)
    return PackedExperts(p13, p2, E, H, I)


@dataclasses.dataclass
class MoEBuffers:
    """Intermediates of one layer call (kept for inspection by tests)."""

    logits: torch.Tensor
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    sorted_ids: torch.Tensor
    block_expert: torch.Tensor
    expert_counts: torch.Tensor
    num_padded: torch.Tensor
    workspace: Optional[torch.Tensor]
    act: torch.Tensor
    y: torch.Tensor
    out: torch.Tensor
    block_m: int
    cap: int
    counters: Optional[torch.Tensor] = None  # zeroed arrival counters of the fused down + combine


def allocate(T: int, H: int, E: int, k: int, I: int, device, block_m: Optional[int] = None,
             out_dtype=torch.bfloat16, y_dtype=torch.float16) -> MoEBuffers:
    """Buffers of one layer call. ``y_dtype`` (fp16 or fp32) is the stored
    precision of the expert outputs between the down GEMM and the combine."""
    if block_m is None:
        block_m = _lib.moe_pick_block_m(T, k, E)
    cap = _lib.moe_align_capacity(T, k, E, block_m)
    if cap < 0:
        raise ValueError("invalid (T, k, E, block_m)")
    ws_bytes = _lib.moe_align_workspace_bytes(T, k, E, block_m)
    i32 = dict(dtype=torch.int32, device=device)
    return MoEBuffers(
        logits=torch.empty((T, E), dtype=torch.float32, device=device),
        topk_ids=torch.empty((T, k), **i32),
        topk_weights=torch.empty((T, k), dtype=torch.float32, device=device),
        sorted_ids=torch.empty((cap,), **i32),
        block_expert=torch.empty((cap // block_m,), **i32),
        expert_counts=torch.empty((E,), **i32),
        num_padded=torch.empty((1,), **i32),
        workspace=torch.empty((ws_bytes,), dtype=torch.uint8, device=device) if ws_bytes else None,
        act=torch.empty((cap, I), dtype=torch.bfloat16, device=device),
        y=torch.empty((T * k, H), dtype=y_dtype, device=device),
        out=torch.empty((T, H), dtype=out_dtype, device=device),
        block_m=block_m,
        cap=cap,
        counters=torch.zeros((max(0, _lib.moe_combine_counter_count(T, H)),), dtype=torch.int32, device=device),
    )


def check_buffers(b: MoEBuffers, T: int, H: int, E: int, k: int, I: int, device) -> None:
    """Raise ValueError unless ``b`` was allocated for this call's (T, H, E,
    k, I) on ``device`` (a buffer from another shape would be written out of
    bounds by the kernels, which take bare pointers)."""
    cap = _lib.moe_align_capacity(T, k, E, b.block_m)
    if cap < 0 or b.cap != cap:
        raise ValueError(f"buffers hold cap={b.cap} rows, the call needs moe_align_capacity(T={T}, k={k}, E={E}, "
                         f"block_m={b.block_m}) = {cap}")
    want = {
        "logits": (T, E), "topk_ids": (T, k), "topk_weights": (T, k), "sorted_ids": (cap,),
        "block_expert": (cap // b.block_m,), "expert_counts": (E,), "num_padded": (1,), "act": (cap, I),
        "y": (T * k, H), "out": (T, H),
    }
    for name, shape in want.items():
        t = getattr(b, name)
        if tuple(t.shape) != shape:
            raise ValueError(f"buffers.{name} has shape {tuple(t.shape)}, the call needs {shape}")
        if t.device != torch.device(device):
            raise ValueError(f"buffers.{name} is on {t.device}, x on {device}")
    if b.counters is not None and b.counters.numel() < _lib.moe_combine_counter_count(T, H):
        raise ValueError("buffers.counters is too small for this call")
    ws = _lib.moe_align_workspace_bytes(T, k, E, b.block_m)
    have = 0 if b.workspace is None else b.workspace.numel() * b.workspace.element_size()
    if have < ws:
        raise ValueError(f"buffers.workspace holds {have} bytes, the call needs {ws}")


def moe_layer(x: torch.Tensor, w_router: torch.Tensor, w13: Optional[torch.Tensor] = None,
              w2: Optional[torch.Tensor] = None, *, top_k: int, norm_topk_prob: bool = True,
              router_bias: Optional[torch.Tensor] = None, packed: Optional[PackedExperts] = None,
              block_m: Optional[int] = None, out_dtype=torch.bfloat16, y_dtype=torch.float16,
              buffers: Optional[MoEBuffers] = None, fused_combine: bool = False, stream=None) -> torch.Tensor:
    """out[T, H] = sparse MoE layer of x[T, H] (no residual).

    ``fused_combine``: run the down projection and the weighted combine as
    one launch (moe_grouped_gemm_down_combine; same output bits) instead of
    moe_grouped_gemm_down followed by moe_combine.

    x [T, H], w_router [E, H]: bf16 on the GPU; router_bias [E] fp32 or None.
    Expert weights either as ``packed`` (from pack_experts, the fast path)
    or as row-major w13 [E, 2I, H] (gate rows, then up rows) and w2 [E, H, I],
    which are then packed on every call. ``y_dtype`` (fp16 or fp32) is the
    stored precision of the expert outputs (ignored when ``buffers`` is
    given: its y decides)."""
    if packed is None:
        if w13 is None or w2 is None:
            raise ValueError("pass packed=pack_experts(w13, w2) or the row-major w13 and w2")
        if w13.dim() != 3 or w2.dim() != 3:
            raise ValueError("w13 [E,2I,H] and w2 [E,H,I] expected")
        if w13.shape[0] != w2.shape[0] or w13.shape[2] != w2.shape[1] or w13.shape[1] != 2 * w2.shape[2]:
            raise ValueError(f"shape mismatch: w13 {tuple(w13.shape)}, w2 {tuple(w2.shape)}")
        packed = pack_experts(w13, w2, stream)
    if x.dim() != 2 or w_router.dim() != 2:
        raise ValueError("x [T,H] and w_router [E,H] expected")
    T, H = x.shape
    E = w_router.shape[0]
    I = packed.intermediate_size
    if w_router.shape[1] != H or packed.num_experts != E or packed.hidden_size != H:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_router {tuple(w_router.shape)}, "
                         f"experts E={packed.num_experts} H={packed.hidden_size} I={I}")
    w13p, w2p = packed.w13, packed.w2
    k = int(top_k)
    for name, t in (("w_router", w_router), ("router_bias", router_bias), ("packed w13", w13p), ("packed w2", w2p)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
    if buffers is not None:
        check_buffers(buffers, T, H, E, k, I, x.device)
        b = buffers
    else:
        b = allocate(T, H, E, k, I, x.device, block_m, out_dtype, y_dtype)
    s = _lib._stream(stream, x)
    _lib.moe_route(x, w_router, router_bias, b.logits, b.topk_ids, b.topk_weights, T, H, E, k, norm_topk_prob, s)
    _lib.moe_align_by_expert(b.topk_ids, T, k, E, b.block_m, b.sorted_ids, b.block_expert, b.expert_counts,
                             b.num_padded, b.workspace, s)
    _lib.moe_grouped_gemm_gate_up_silu(x, w13p, b.sorted_ids, b.block_expert, b.num_padded, T, k, H, I, E, b.block_m,
                                       b.cap, b.act, s)
    if fused_combine:
        _lib.moe_grouped_gemm_down_combine(b.act, w2p, b.sorted_ids, b.block_expert, b.num_padded, b.topk_weights, T, k,
                                           H, I, E, b.block_m, b.cap, b.y, b.counters, b.out, s)
    else:
        _lib.moe_grouped_gemm_down(b.act, w2p, b.sorted_ids, b.block_expert, b.num_padded, T, k, H, I, E, b.block_m,
                                   b.cap, b.y, s)
        _lib.moe_combine(b.y, b.topk_weights, T, k, H, b.out, s)
    return b.out


def moe_layer_with_norm(x: torch.Tensor, residual: Optional[torch.Tensor], norm_weight: torch.Tensor,
                        w_router: torch.Tensor, *, top_k: int, packed: PackedExperts, eps: float = 1e-6,
                        norm_topk_prob: bool = True, router_bias: Optional[torch.Tensor] = None,
                        block_m: Optional[int] = None, out_dtype=torch.bfloat16, y_dtype=torch.float16,
                        buffers: Optional[MoEBuffers] = None, stream=None):
    """The decoder's post-attention residual add + RMSNorm and the MoE layer:
    ``residual' = residual + x`` (``x`` when ``residual`` is None, the first
    layer), ``h = rmsnorm(residual') * norm_weight``, ``out = moe(h)``. The
    add and norm run inside the router kernel (moe_fused_add_rmsnorm_route);
    the grouped GEMMs read ``h``. Returns (out, residual', h)."""
    if x.dim() != 2:
        raise ValueError("x [T,H] expected")
    T, H = x.shape
    E = w_router.shape[0]
    I = packed.intermediate_size
    k = int(top_k)
    if buffers is not None:
        check_buffers(buffers, T, H, E, k, I, x.device)
        b = buffers
    else:
        b = allocate(T, H, E, k, I, x.device, block_m, out_dtype, y_dtype)
    h = torch.empty_like(x)
    res_out = torch.empty_like(x)
    s = _lib._stream(stream, x)
    _lib.moe_fused_add_rmsnorm_route(x, residual, norm_weight, eps, residual is not None, h, res_out, w_router,
                                     router_bias, b.logits, b.topk_ids, b.topk_weights, T, H, E, k, norm_topk_prob, s)
    _lib.moe_align_by_expert(b.topk_ids, T, k, E, b.block_m, b.sorted_ids, b.block_expert, b.expert_counts,
                             b.num_padded, b.workspace, s)
    _lib.moe_grouped_gemm_gate_up_silu(h, packed.w13, b.sorted_ids, b.block_expert, b.num_padded, T, k, H, I, E,
                                       b.block_m, b.cap, b.act, s)
    _lib.moe_grouped_gemm_down(b.act, packed.w2, b.sorted_ids, b.block_expert, b.num_padded, T, k, H, I, E,
                               b.block_m, b.cap, b.y, s)
    _lib.moe_combine(b.y, b.topk_weights, T, k, H, b.out, s)
    return b.out, res_out, h


def dense_down_block_m(T: int, H: int, block_m: int, cus: int) -> int:
    """Row-block size of the down projection in the single-expert path.

    With one expert the grouping is the identity at every block size (row r
    of the sorted order is token r, the pad rows follow), so the two
    projections may use different row blocks. The down projection's N = H is
    narrow: when its 128-row tiles (512 columns wide) would not give every
    compute unit one, 64-row blocks (64x256 tiles, two per CU) are used
    instead (T = 4096, H = 1024: 66 -> 37 us, gate/up staying at 128 rows)."""
    if block_m >= 128 and -(-T // 128) * -(-H // 512) < cus:
        return 64
    return block_m


def gated_mlp(x: torch.Tensor, packed: PackedExperts, *, block_m: Optional[int] = None, out_dtype=torch.bfloat16,
              y_dtype=torch.float16, stream=None) -> torch.Tensor:
    """Dense SwiGLU GatedMLP (down(silu(gate(x)) * up(x)), the "Models and
    weight loading" page's GatedMLP) through the same grouped GEMMs: every
    token is routed to the single expert of ``packed`` (num_experts == 1)
    with weight 1, so the grouping is the identity and the combine is a copy
    to the output dtype. Used for dense layers and mlp_only_layers."""
    if packed.num_experts != 1:
        raise ValueError("gated_mlp needs a single packed expert (E = 1)")
    if x.dim() != 2 or x.shape[1] != packed.hidden_size:
        raise ValueError(f"x must be [T, {packed.hidden_size}]")
    T, H = x.shape
    I = packed.intermediate_size
    b = allocate(T, H, 1, 1, I, x.device, block_m, out_dtype, y_dtype)
    s = _lib._stream(stream, x)
    ids = torch.zeros((T, 1), dtype=torch.int32, device=x.device)
    ones = torch.ones((T, 1), dtype=torch.float32, device=x.device)
    _lib.moe_align_by_expert(ids, T, 1, 1, b.block_m, b.sorted_ids, b.block_expert, b.expert_counts, b.num_padded,
                             b.workspace, s)
    _lib.moe_grouped_gemm_gate_up_silu(x, packed.w13, b.sorted_ids, b.block_expert, b.num_padded, T, 1, H, I, 1,
                                       b.block_m, b.cap, b.act, s)
    cus = torch.cuda.get_device_properties(x.device).multi_processor_count if x.is_cuda else 0
    down_bm = b.block_m if block_m is not None else dense_down_block_m(T, H, b.block_m, cus)
    if down_bm == b.block_m:
        _lib.moe_grouped_gemm_down(b.act, packed.w2, b.sorted_ids, b.block_expert, b.num_padded, T, 1, H, I, 1,
                                   b.block_m, b.cap, b.y, s)
    else:
        # the grouping at the finer block size (the identity again), from the
        # library's own grouping call; act's rows are the same rows and hold
        # at least that grouping's capacity
        cap = _lib.moe_align_capacity(T, 1, 1, down_bm)
        assert cap <= b.cap and b.cap % down_bm == 0
        i32 = dict(dtype=torch.int32, device=x.device)
        sorted_ids, block_expert = torch.empty((cap,), **i32), torch.empty((cap // down_bm,), **i32)
        counts, num_padded = torch.empty((1,), **i32), torch.empty((1,), **i32)
        ws_bytes = _lib.moe_align_workspace_bytes(T, 1, 1, down_bm)
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=x.device) if ws_bytes else None
        _lib.moe_align_by_expert(ids, T, 1, 1, down_bm, sorted_ids, block_expert, counts, num_padded, ws, s)
        _lib.moe_grouped_gemm_down(b.act, packed.w2, sorted_ids, block_expert, num_padded, T, 1, H, I, 1, down_bm,
                                   cap, b.y, s)
    _lib.moe_combine(b.y, ones, T, 1, H, b.out, s)
    return b.out
