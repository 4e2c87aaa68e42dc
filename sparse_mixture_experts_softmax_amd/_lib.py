"""ctypes binding of libmoe_mi355x.so (the C ABI in include/moe_mi355x.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. The functions keep the C names; device buffers are torch tensors
(checked for device, dtype and contiguity here), sizes are Python ints, and
``stream`` defaults to torch's current stream on the tensors' device. A
nonzero status raises ``MoEError`` with the library's message. There is no
fallback: if the library is missing or does not load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB names another build of the library (e.g. the host-sanitizer
# test build); there is still no fallback when it is missing.
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_WORKSPACE = -4
MOE_DTYPE_BF16 = 0
MOE_DTYPE_FP32 = 1
MOE_DTYPE_FP16 = 2
MOE_OUT_BF16 = MOE_DTYPE_BF16
MOE_OUT_FP32 = MOE_DTYPE_FP32
MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES = 262144
_Y_DTYPES = {torch.float16: MOE_DTYPE_FP16, torch.float32: MOE_DTYPE_FP32}

EXPORTS = (
    "moe_abi_version",
    "moe_last_error",
    "moe_route",
    "moe_align_capacity",
    "moe_align_workspace_bytes",
    "moe_align_by_expert",
    "moe_align_by_expert_noalloc",
    "moe_grouped_gemm_gate_up_silu",
    "moe_grouped_gemm_down",
    "moe_combine",
    "moe_grouped_gemm_down_combine",
    "moe_combine_counter_count",
    "moe_pick_block_m",
    "moe_packed_weight_bytes",
    "moe_pack_weights",
    "moe_fused_add_rmsnorm",
    "moe_fused_add_rmsnorm_route",
)


class MoEError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class LibraryMissing(RuntimeError):
    pass


_lib = None


def lib():
    """The loaded library (raises LibraryMissing if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is not built; run python -m sparse_mixture_experts_softmax_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_abi_version.argtypes, L.moe_abi_version.restype = [], ctypes.c_int
        L.moe_last_error.argtypes, L.moe_last_error.restype = [], ctypes.c_char_p
        L.moe_route.argtypes = [p, p, p, p, p, p, i64, i32, i32, i32, i32, p]
        L.moe_align_capacity.argtypes, L.moe_align_capacity.restype = [i64, i32, i32, i32], i64
        L.moe_align_workspace_bytes.argtypes, L.moe_align_workspace_bytes.restype = [i64, i32, i32, i32], sz
        L.moe_align_by_expert.argtypes = [p, i64, i32, i32, i32, p, p, p, p, p, sz, p]
        L.moe_align_by_expert_noalloc.argtypes = [p, i64, i32, i32, i32, p, p, p, p, p]
        L.moe_align_by_expert_noalloc.restype = ctypes.c_int
        L.moe_grouped_gemm_gate_up_silu.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i32, i32, i64, p, p]
        L.moe_grouped_gemm_down.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i32, i32, i64, p, i32, p]
        L.moe_combine.argtypes = [p, i32, p, i64, i32, i32, p, i32, p]
        L.moe_grouped_gemm_down_combine.argtypes = [p, p, p, p, p, p, i64, i32, i32, i32, i32, i32, i64, p, i32, p, p,
                                                     i32, p]
        L.moe_grouped_gemm_down_combine.restype = ctypes.c_int
        L.moe_combine_counter_count.argtypes, L.moe_combine_counter_count.restype = [i64, i32], i64
        L.moe_pick_block_m.argtypes, L.moe_pick_block_m.restype = [i64, i32, i32], i32
        L.moe_packed_weight_bytes.argtypes, L.moe_packed_weight_bytes.restype = [i32, i32, i32], sz
        L.moe_pack_weights.argtypes, L.moe_pack_weights.restype = [p, p, i32, i32, i32, i32, p], ctypes.c_int
        L.moe_fused_add_rmsnorm.argtypes = [p, p, p, i64, i32, ctypes.c_float, i32, p]
        L.moe_fused_add_rmsnorm.restype = ctypes.c_int
        L.moe_fused_add_rmsnorm_route.argtypes = [p, p, p, ctypes.c_float, i32, p, p, p, p, p, p, p, i64, i32, i32,
                                                  i32, i32, p]
        L.moe_fused_add_rmsnorm_route.restype = ctypes.c_int
        for name in ("moe_route", "moe_align_by_expert", "moe_grouped_gemm_gate_up_silu", "moe_grouped_gemm_down",
                     "moe_combine"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoEError(rc, lib().moe_last_error().decode())


def _dev(t: Optional[torch.Tensor], dtype, name: str, optional: bool = False, numel: int = 0, device=None):
    """data pointer of a contiguous GPU tensor of the given dtype (or None)."""
    return _ptrs((t, dtype, name, optional, numel), device=device)[0]


def _ptrs(*specs, device=None):
    """Data pointers of a call's tensors, each spec being (tensor, dtype,
    name, optional, numel). ``numel`` is the least number of elements the
    call reads or writes through that tensor (the C ABI takes bare pointers
    and cannot check sizes, so a short buffer would become an out-of-bounds
    device access). Every tensor's type, size and layout are checked before
    any tensor's device, so the checks run the same on a machine without a
    GPU. All tensors must be on one GPU (``device`` if given)."""
    for t, dtype, name, optional, numel in specs:
        if t is None:
            if optional:
                continue
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.numel() < numel:
            raise ValueError(f"{name} has {t.numel()} elements, the call needs at least {numel}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    out = []
    for t, dtype, name, optional, numel in specs:
        if t is None:
            out.append(None)
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {device}")
        out.append(t.data_ptr() if t.numel() else None)
    return out


def _nonneg(**sizes):
    for name, v in sizes.items():
        if int(v) < 0:
            raise ValueError(f"{name} must be non-negative, got {v}")


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_route(x, w_router, router_bias, logits, topk_ids, topk_weights, T: int, H: int, E: int, k: int,
              norm_topk_prob: bool, stream=None):
    """Router linear + softmax + top-k (+ renorm). ``x=None``: logits are an input."""
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _nonneg(T=T, H=H, E=E, k=k)
    args = _ptrs(
        (x, bf, "x", True, T * H),
        (w_router, bf, "w_router", x is None, E * H if x is not None else 0),
        (router_bias, f32, "router_bias", True, E),
        (logits, f32, "logits", False, T * E),
        (topk_ids, i32, "topk_ids", False, T * k),
        (topk_weights, f32, "topk_weights", False, T * k),
    )
    _check(lib().moe_route(*args, T, H, E, k, int(bool(norm_topk_prob)), _stream(stream, logits)))


def moe_align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return lib().moe_align_capacity(T, k, E, block_m)


def moe_align_workspace_bytes(T: int, k: int, E: int, block_m: int) -> int:
    return lib().moe_align_workspace_bytes(T, k, E, block_m)


def moe_pick_block_m(T: int, k: int, E: int) -> int:
    return lib().moe_pick_block_m(T, k, E)


def moe_packed_weight_bytes(E: int, N: int, K: int) -> int:
    return lib().moe_packed_weight_bytes(E, N, K)


def moe_pack_weights(w, w_packed, E: int, N: int, K: int, gated: bool, stream=None):
    """Row-major [E, N, K] bf16 -> the GEMMs' fragment layout (same size)."""
    bf = torch.bfloat16
    _nonneg(E=E, N=N, K=K)
    pw, pp = _ptrs((w, bf, "w", False, E * N * K), (w_packed, bf, "w_packed", False, E * N * K))
    _check(lib().moe_pack_weights(pw, pp, E, N, K, int(bool(gated)), _stream(stream, w)))


def moe_fused_add_rmsnorm(x, residual, weight, T: int, H: int, eps: float, has_residual: bool, stream=None):
    """In place: residual <- residual + x (or x), x <- rmsnorm(residual)."""
    bf = torch.bfloat16
    _nonneg(T=T, H=H)
    px, pr, pw = _ptrs((x, bf, "x", False, T * H), (residual, bf, "residual", False, T * H),
                       (weight, bf, "weight", False, H))
    _check(lib().moe_fused_add_rmsnorm(px, pr, pw, T, H, float(eps), int(bool(has_residual)), _stream(stream, x)))


def moe_fused_add_rmsnorm_route(x, residual, norm_weight, eps: float, has_residual: bool, x_out, residual_out,
                                w_router, router_bias, logits, topk_ids, topk_weights, T: int, H: int, E: int, k: int,
                                norm_topk_prob: bool, stream=None):
    """residual_out <- residual + x (or x), x_out <- rmsnorm(residual_out),
    then the router on x_out, in one pass over the rows (outputs may not
    overlap the inputs)."""
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _nonneg(T=T, H=H, E=E, k=k)
    p = _ptrs((x, bf, "x", False, T * H), (residual, bf, "residual", not has_residual, T * H),
              (norm_weight, bf, "norm_weight", False, H), (x_out, bf, "x_out", False, T * H),
              (residual_out, bf, "residual_out", False, T * H), (w_router, bf, "w_router", False, E * H),
              (router_bias, f32, "router_bias", True, E), (logits, f32, "logits", False, T * E),
              (topk_ids, i32, "topk_ids", False, T * k), (topk_weights, f32, "topk_weights", False, T * k))
    _check(lib().moe_fused_add_rmsnorm_route(p[0], p[1] if has_residual else None, p[2], float(eps),
                                             int(bool(has_residual)), p[3], p[4], p[5], p[6], p[7], p[8], p[9], T, H,
                                             E, k, int(bool(norm_topk_prob)), _stream(stream, x)))


def moe_align_by_expert(topk_ids, T: int, k: int, E: int, block_m: int, sorted_ids, block_expert, expert_counts,
                        num_padded, workspace=None, stream=None):
    i32 = torch.int32
    _nonneg(T=T, k=k, E=E)
    cap = max(0, lib().moe_align_capacity(T, k, E, block_m))
    ws_bytes = 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    p = _ptrs((topk_ids, i32, "topk_ids", False, T * k), (sorted_ids, i32, "sorted_ids", False, cap),
              (block_expert, i32, "block_expert", False, cap // max(block_m, 1)),
              (expert_counts, i32, "expert_counts", False, E), (num_padded, i32, "num_padded", False, 1),
              (workspace, workspace.dtype if workspace is not None else None, "workspace", True, 0))
    _check(lib().moe_align_by_expert(p[0], T, k, E, block_m, p[1], p[2], p[3], p[4], p[5], ws_bytes,
                                     _stream(stream, topk_ids)))


def moe_grouped_gemm_gate_up_silu(x, w13, sorted_ids, block_expert, num_padded, T: int, k: int, H: int, I: int,
                                  E: int, block_m: int, cap: int, act, stream=None):
    bf, i32 = torch.bfloat16, torch.int32
    _nonneg(T=T, k=k, H=H, I=I, E=E, cap=cap)
    bm = max(block_m, 1)
    p = _ptrs((x, bf, "x", False, T * H), (w13, bf, "w13", False, E * 2 * I * H),
              (sorted_ids, i32, "sorted_ids", False, cap), (block_expert, i32, "block_expert", False, cap // bm),
              (num_padded, i32, "num_padded", False, 1), (act, bf, "act", False, cap * I))
    _check(lib().moe_grouped_gemm_gate_up_silu(p[0], p[1], p[2], p[3], p[4], T, k, H, I, E, block_m, cap, p[5],
                                               _stream(stream, x)))


def _y_dtype(y) -> int:
    if y is None or y.dtype not in _Y_DTYPES:
        raise TypeError("y must be a fp16 or fp32 tensor")
    return _Y_DTYPES[y.dtype]


def moe_grouped_gemm_down(act, w2, sorted_ids, block_expert, num_padded, T: int, k: int, H: int, I: int, E: int,
                          block_m: int, cap: int, y, stream=None):
    """``y`` dtype (fp16 or fp32) selects the stored precision of y."""
    bf, i32 = torch.bfloat16, torch.int32
    yd = _y_dtype(y)
    _nonneg(T=T, k=k, H=H, I=I, E=E, cap=cap)
    bm = max(block_m, 1)
    p = _ptrs((act, bf, "act", False, cap * I), (w2, bf, "w2", False, E * H * I),
              (sorted_ids, i32, "sorted_ids", False, cap), (block_expert, i32, "block_expert", False, cap // bm),
              (num_padded, i32, "num_padded", False, 1), (y, y.dtype, "y", False, T * k * H))
    _check(lib().moe_grouped_gemm_down(p[0], p[1], p[2], p[3], p[4], T, k, H, I, E, block_m, cap, p[5], yd,
                                       _stream(stream, act)))


def moe_combine(y, topk_weights, T: int, k: int, H: int, out, stream=None):
    """``y`` dtype (fp16 or fp32) is the stored y; ``out`` dtype (bf16 or
    fp32) selects the output precision."""
    if out is None or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be a bf16 or fp32 tensor")
    od = MOE_OUT_FP32 if out.dtype == torch.float32 else MOE_OUT_BF16
    yd = _y_dtype(y)
    _nonneg(T=T, k=k, H=H)
    p = _ptrs((y, y.dtype, "y", False, T * k * H), (topk_weights, torch.float32, "topk_weights", False, T * k),
              (out, out.dtype, "out", False, T * H))
    _check(lib().moe_combine(p[0], yd, p[1], T, k, H, p[2], od, _stream(stream, y)))


def moe_align_noalloc_max_workspace_bytes() -> int:
    """Static scratch of moe_align_by_expert_noalloc (the header's
    MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES)."""
    return MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES


def moe_align_by_expert_noalloc(topk_ids, T: int, k: int, E: int, block_m: int, sorted_ids, block_expert,
                                expert_counts, num_padded, stream=None):
    """moe_align_by_expert with its histograms in the library's static device
    scratch (no workspace, nothing allocated); calls on one GPU must not
    overlap."""
    i32 = torch.int32
    _nonneg(T=T, k=k, E=E)
    cap = max(0, lib().moe_align_capacity(T, k, E, block_m))
    p = _ptrs((topk_ids, i32, "topk_ids", False, T * k), (sorted_ids, i32, "sorted_ids", False, cap),
              (block_expert, i32, "block_expert", False, cap // max(block_m, 1)),
              (expert_counts, i32, "expert_counts", False, E), (num_padded, i32, "num_padded", False, 1))
    _check(lib().moe_align_by_expert_noalloc(p[0], T, k, E, block_m, p[1], p[2], p[3], p[4],
                                             _stream(stream, topk_ids)))


def moe_combine_counter_count(T: int, H: int) -> int:
    return lib().moe_combine_counter_count(T, H)


def moe_grouped_gemm_down_combine(act, w2, sorted_ids, block_expert, num_padded, topk_weights, T: int, k: int, H: int,
                                  I: int, E: int, block_m: int, cap: int, y, counters, out, stream=None):
    """Down projection with the weighted combine fused in. ``y`` (fp16 or
    fp32) holds the expert outputs; ``counters`` (int32, zero, of
    moe_combine_counter_count(T, H) elements) are left zero; ``out`` dtype
    (bf16 or fp32) selects the output precision."""
    if out is None or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be a bf16 or fp32 tensor")
    od = MOE_OUT_FP32 if out.dtype == torch.float32 else MOE_OUT_BF16
    yd = _y_dtype(y)
    bf, i32 = torch.bfloat16, torch.int32
    _nonneg(T=T, k=k, H=H, I=I, E=E, cap=cap)
    bm = max(block_m, 1)
    n_cnt = max(0, lib().moe_combine_counter_count(T, H))
    p = _ptrs((act, bf, "act", False, cap * I), (w2, bf, "w2", False, E * H * I),
              (sorted_ids, i32, "sorted_ids", False, cap), (block_expert, i32, "block_expert", False, cap // bm),
              (num_padded, i32, "num_padded", False, 1), (topk_weights, torch.float32, "topk_weights", False, T * k),
              (y, y.dtype, "y", False, T * k * H), (counters, i32, "counters", False, n_cnt),
              (out, out.dtype, "out", False, T * H))
    _check(lib().moe_grouped_gemm_down_combine(p[0], p[1], p[2], p[3], p[4], p[5], T, k, H, I, E, block_m, cap, p[6],
                                               yd, p[7], p[8], od, _stream(stream, act)))
