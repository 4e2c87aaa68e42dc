"""Fused sparse Mixture-of-Experts layer for AMD Instinct MI355X (gfx950).

Router linear -> softmax -> top-k (optional renormalisation) -> tokens grouped
by expert -> grouped gate/up GEMM with SiLU-and-mul -> grouped down GEMM ->
weighted combine, each a hand-written HIP kernel in libmoe_mi355x.so (C ABI:
include/moe_mi355x.h). This package is the thin Python binding over it.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MOE_DTYPE_BF16,
    MOE_DTYPE_FP16,
    MOE_DTYPE_FP32,
    MOE_ERR_HIP,
    MOE_ERR_INVALID,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    LibraryMissing,
    MoEError,
    lib,
    moe_abi_version,
    moe_align_by_expert,
    moe_align_by_expert_noalloc,
    moe_align_noalloc_max_workspace_bytes,
    moe_align_capacity,
    moe_align_workspace_bytes,
    moe_combine,
    moe_combine_counter_count,
    moe_fused_add_rmsnorm,
    moe_fused_add_rmsnorm_route,
    moe_grouped_gemm_down,
    moe_grouped_gemm_down_combine,
    moe_grouped_gemm_gate_up_silu,
    moe_last_error,
    moe_pack_weights,
    moe_packed_weight_bytes,
    moe_pick_block_m,
    moe_route,
)
from .layer import (  # noqa: F401
    MoEBuffers,
    MoEConfig,
    PackedExperts,
    allocate,
    check_buffers,
    dense_down_block_m,
    gated_mlp,
    moe_layer,
    moe_layer_with_norm,
    pack_experts,
)
