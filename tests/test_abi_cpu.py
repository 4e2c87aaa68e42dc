"""The C-ABI library on a machine without a GPU: it loads, exports every
entry point the header declares, and rejects bad arguments on the host
before enqueueing anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest
import torch

import sparse_mixture_experts_softmax_amd as moe
from sparse_mixture_experts_softmax_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = declared_functions()
    assert len(names) >= 10, names
    for name in names:
        assert hasattr(L, name), f"{name} declared in the header but not exported"
    assert set(names) == set(_lib.EXPORTS)
    assert moe.moe_abi_version() == 3


def test_capacity_and_workspace():
    assert moe.moe_align_capacity(64, 8, 128, 16) == 512 + 128 * 15
    assert moe.moe_align_capacity(16, 2, 8, 16) == 160  # 32 + 8*15 = 152 -> 160
    assert moe.moe_align_capacity(1, 1, 256, 128) == 128
    assert moe.moe_align_capacity(0, 8, 128, 64) == 0
    assert moe.moe_align_capacity(10, 2, 8, 48) == -1
    assert moe.moe_align_capacity(10, 2, 8, 512) == -1
    assert moe.moe_align_capacity(64, 8, 128, 256) == (512 + 128 * 255 + 255) // 256 * 256
    assert moe.moe_align_workspace_bytes(64, 8, 128, 16) == 0  # one tile: no workspace
    assert moe.moe_align_workspace_bytes(16384, 8, 128, 64) == 32 * 128 * 4  # 32 tiles of 4096 pairs
    assert moe.moe_align_workspace_bytes(4096, 8, 128, 64) == 32 * 128 * 4  # 32 tiles of 1024 pairs
    assert moe.moe_align_workspace_bytes(128, 8, 128, 64) == 0  # one tile
    for T, k, E in ((64, 8, 128), (4096, 8, 128), (16, 2, 8)):
        assert moe.moe_pick_block_m(T, k, E) in (16, 32, 64, 128)
    # the measured crossovers, in rows per expert (T * k / E): below 16 | up to 60
    picks = {64: 16, 240: 16, 255: 16, 256: 64, 352: 64, 512: 64, 960: 64, 976: 128, 4096: 128}
    for T, bm in picks.items():
        assert moe.moe_pick_block_m(T, 8, 128) == bm, T
    assert moe.moe_pick_block_m(-1, 8, 128) == -1 and moe.moe_pick_block_m(4, 0, 8) == -1
    # single-expert path: 64-row down blocks only while 128-row tiles would
    # leave compute units idle
    assert moe.dense_down_block_m(4096, 1024, 128, 256) == 64
    assert moe.dense_down_block_m(65536, 1024, 128, 256) == 128
    assert moe.dense_down_block_m(4096, 1024, 16, 256) == 16


def _raw():
    return moe.lib()


NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation


@pytest.mark.parametrize(
    "args,code",
    [
        # moe_route(x, wr, bias, logits, ids, w, T, H, E, k, norm, stream)
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 4, 64, 300, 2, 1, NULL), _lib.MOE_ERR_UNSUPPORTED),
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 4, 64, 8, 9, 1, NULL), _lib.MOE_ERR_UNSUPPORTED),
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 4, 64, 64, 33, 1, NULL), _lib.MOE_ERR_UNSUPPORTED),
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 4, 96, 8, 2, 1, NULL), _lib.MOE_ERR_UNSUPPORTED),
        ((FAKE, NULL, NULL, FAKE, FAKE, FAKE, 4, 64, 8, 2, 1, NULL), _lib.MOE_ERR_INVALID),
        ((FAKE, FAKE, NULL, NULL, FAKE, FAKE, 4, 64, 8, 2, 1, NULL), _lib.MOE_ERR_INVALID),
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, -1, 64, 8, 2, 1, NULL), _lib.MOE_ERR_INVALID),
        ((FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 0, 64, 8, 2, 1, NULL), _lib.MOE_OK),
        ((NULL, NULL, NULL, FAKE, FAKE, FAKE, 0, 0, 8, 2, 1, NULL), _lib.MOE_OK),
    ],
)
def test_route_validation(args, code):
    assert _raw().moe_route(*args) == code
    if code:
        assert moe.moe_last_error().startswith("moe_route")


def test_align_validation():
    L = _raw()
    # (ids, T, k, E, block_m, sorted, blk, counts, npad, ws, ws_bytes, stream)
    assert L.moe_align_by_expert(FAKE, 16, 2, 8, 48, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_align_by_expert(FAKE, 16, 9, 8, 16, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_align_by_expert(NULL, 16, 2, 8, 16, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == _lib.MOE_ERR_INVALID
    # several tiles need a workspace
    assert L.moe_align_by_expert(FAKE, 4096, 8, 128, 64, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_align_by_expert(FAKE, 4096, 8, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 100, NULL) == _lib.MOE_ERR_WORKSPACE
    assert "workspace" in moe.moe_last_error()
    assert L.moe_align_by_expert(NULL, 0, 2, 8, 16, NULL, NULL, NULL, NULL, NULL, 0, NULL) == _lib.MOE_OK


def test_gemm_validation():
    L = _raw()
    F16 = _lib.MOE_DTYPE_FP16
    calls = (lambda *a: L.moe_grouped_gemm_gate_up_silu(*a[:-1], NULL),
             lambda *a: L.moe_grouped_gemm_down(*a[:-1], F16, NULL))
    for fn in calls:
        # (a, w, sorted, blk, npad, T, k, H, I, E, block_m, cap, out, stream)
        cap = moe.moe_align_capacity(16, 2, 8, 16)
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 48, 8, 16, cap, FAKE, NULL) == _lib.MOE_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 100, 32, 8, 16, cap, FAKE, NULL) == _lib.MOE_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 32, 8, 24, cap, FAKE, NULL) == _lib.MOE_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 32, 8, 16, cap - 16, FAKE, NULL) == _lib.MOE_ERR_WORKSPACE
        assert fn(FAKE, NULL, FAKE, FAKE, FAKE, 16, 2, 64, 32, 8, 16, cap, FAKE, NULL) == _lib.MOE_ERR_INVALID
        misaligned = ctypes.c_void_p(0x1002)
        assert fn(misaligned, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 32, 8, 16, cap, FAKE, NULL) == _lib.MOE_ERR_INVALID
        assert fn(NULL, NULL, NULL, NULL, NULL, 0, 2, 64, 32, 8, 16, 0, NULL, NULL) == _lib.MOE_OK
    # block_m 64/128: activations over 4 GiB are refused before any launch
    # (x of T=2^21 tokens at H=2048 is 8 GiB)
    big_T = 1 << 21
    cap = moe.moe_align_capacity(big_T, 2, 8, 128)
    assert L.moe_grouped_gemm_gate_up_silu(FAKE, FAKE, FAKE, FAKE, FAKE, big_T, 2, 2048, 32, 8, 128, cap, FAKE,
                                           NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert "4 GiB" in moe.moe_last_error()
    assert L.moe_grouped_gemm_down(FAKE, FAKE, FAKE, FAKE, FAKE, big_T, 2, 64, 2048, 8, 128, cap, FAKE, F16,
                                   NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert "4 GiB" in moe.moe_last_error()
    # y is fp16 or fp32, nothing else (bf16 included)
    cap = moe.moe_align_capacity(16, 2, 8, 16)
    for bad in (_lib.MOE_DTYPE_BF16, 3, -1):
        assert L.moe_grouped_gemm_down(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, 64, 32, 8, 16, cap, FAKE, bad,
                                       NULL) == _lib.MOE_ERR_INVALID
        assert "y_dtype" in moe.moe_last_error()


def test_pack_validation():
    L = _raw()
    assert moe.moe_packed_weight_bytes(128, 1536, 2048) == 128 * 1536 * 2048 * 2
    assert moe.moe_packed_weight_bytes(2, 24, 64) == 0
    other = ctypes.c_void_p(0x2000)
    assert L.moe_pack_weights(FAKE, other, 2, 24, 64, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(FAKE, other, 2, 32, 48, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(FAKE, other, 2, 48, 64, 1, NULL) == _lib.MOE_ERR_UNSUPPORTED  # gated needs I % 16
    assert L.moe_pack_weights(FAKE, FAKE, 2, 32, 64, 0, NULL) == _lib.MOE_ERR_INVALID  # in place
    assert L.moe_pack_weights(NULL, other, 2, 32, 64, 0, NULL) == _lib.MOE_ERR_INVALID


def test_rmsnorm_validation():
    L = _raw()
    other = ctypes.c_void_p(0x2000)
    f = L.moe_fused_add_rmsnorm
    assert f(FAKE, other, FAKE, 4, 12, ctypes.c_float(1e-6), 1, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert f(FAKE, other, FAKE, 4, 8 * 2048 + 8, ctypes.c_float(1e-6), 1, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert f(FAKE, other, FAKE, 4, 64, ctypes.c_float(-1.0), 1, NULL) == _lib.MOE_ERR_INVALID
    assert f(FAKE, FAKE, FAKE, 4, 64, ctypes.c_float(1e-6), 1, NULL) == _lib.MOE_ERR_INVALID  # aliasing
    assert f(NULL, other, FAKE, 4, 64, ctypes.c_float(1e-6), 1, NULL) == _lib.MOE_ERR_INVALID
    assert f(NULL, NULL, NULL, 0, 64, ctypes.c_float(1e-6), 1, NULL) == _lib.MOE_OK


def test_combine_validation():
    L = _raw()
    F16, F32 = _lib.MOE_DTYPE_FP16, _lib.MOE_DTYPE_FP32
    assert L.moe_combine(FAKE, F16, FAKE, 4, 2, 64, FAKE, 7, NULL) == _lib.MOE_ERR_INVALID
    assert L.moe_combine(FAKE, _lib.MOE_DTYPE_BF16, FAKE, 4, 2, 64, FAKE, 0, NULL) == _lib.MOE_ERR_INVALID
    assert "y_dtype" in moe.moe_last_error()
    assert L.moe_combine(FAKE, F16, FAKE, 4, 33, 64, FAKE, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(FAKE, F32, FAKE, 4, 2, 32, FAKE, 0, NULL) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(NULL, F16, FAKE, 4, 2, 64, FAKE, 0, NULL) == _lib.MOE_ERR_INVALID
    assert L.moe_combine(NULL, F32, NULL, 0, 2, 64, NULL, 0, NULL) == _lib.MOE_OK


def test_python_binding_rejects_host_tensors_and_wrong_dtypes():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_combine(torch.zeros(8, 64), torch.zeros(4, 2), 4, 2, 64, x)
    with pytest.raises(TypeError):
        moe.moe_combine(torch.zeros(8, 64, dtype=torch.bfloat16), torch.zeros(4, 2), 4, 2, 64, x)
    with pytest.raises(ValueError, match="Unsupported activation"):
        moe.MoEConfig(64, 8, 2, 32, hidden_act="gelu")


def test_status_raises_with_message():
    with pytest.raises(moe.MoEError, match="E=300"):
        _lib._check(_raw().moe_route(FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 4, 64, 300, 2, 1, NULL))


def test_header_abi_version_matches_library():
    """build() checks the loaded library against the header's version."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "include", "moe_mi355x.h")) as fh:
        header_version = int(re.search(r"#define MOE_ABI_VERSION (\d+)", fh.read()).group(1))
    assert moe.moe_abi_version() == header_version


def test_build_rejects_scratch():
    # the build fails when a kernel's resource-usage remark reports scratch
    from sparse_mixture_experts_softmax_amd import build
    clean = ("a.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
             "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    spill = clean + ("a.hip:9:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]\n"
                     "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build._scratch_users(clean) == []
    assert build._scratch_users(spill) == ["_Z1jv (36 bytes/lane)"]


# ----------------------------------------------------------------------------
# The Python binding checks buffer sizes before anything reaches the C ABI
# (which takes bare pointers and cannot): a short buffer raises ValueError.
# ----------------------------------------------------------------------------
def _t(n, dtype=torch.int32):
    return torch.zeros(n, dtype=dtype)


@pytest.mark.parametrize("which", ["topk_ids", "sorted_ids", "block_expert", "expert_counts", "num_padded"])
def test_align_binding_rejects_short_buffers(which):
    T, k, E, bm = 100, 4, 16, 32
    cap = moe.moe_align_capacity(T, k, E, bm)
    bufs = dict(topk_ids=_t(T * k), sorted_ids=_t(cap), block_expert=_t(cap // bm), expert_counts=_t(E),
                num_padded=_t(1))
    bufs[which] = _t(bufs[which].numel() - 1)
    with pytest.raises(ValueError, match=which):
        moe.moe_align_by_expert(bufs["topk_ids"], T, k, E, bm, bufs["sorted_ids"], bufs["block_expert"],
                                bufs["expert_counts"], bufs["num_padded"])


@pytest.mark.parametrize("which", ["x", "w_router", "logits", "topk_ids", "topk_weights"])
def test_route_binding_rejects_short_buffers(which):
    T, H, E, k = 10, 64, 8, 2
    bf, f32 = torch.bfloat16, torch.float32
    bufs = dict(x=_t(T * H, bf), w_router=_t(E * H, bf), logits=_t(T * E, f32), topk_ids=_t(T * k),
                topk_weights=_t(T * k, f32))
    bufs[which] = _t(bufs[which].numel() - 1, bufs[which].dtype)
    with pytest.raises(ValueError, match=which):
        moe.moe_route(bufs["x"], bufs["w_router"], None, bufs["logits"], bufs["topk_ids"], bufs["topk_weights"], T, H,
                      E, k, True)


@pytest.mark.parametrize("which", ["x", "w13", "sorted_ids", "block_expert", "act"])
def test_gate_up_binding_rejects_short_buffers(which):
    T, H, E, k, I, bm = 10, 64, 8, 2, 32, 16
    cap = moe.moe_align_capacity(T, k, E, bm)
    bf = torch.bfloat16
    bufs = dict(x=_t(T * H, bf), w13=_t(E * 2 * I * H, bf), sorted_ids=_t(cap), block_expert=_t(cap // bm),
                num_padded=_t(1), act=_t(cap * I, bf))
    bufs[which] = _t(bufs[which].numel() - 1, bufs[which].dtype)
    with pytest.raises(ValueError, match=which):
        moe.moe_grouped_gemm_gate_up_silu(bufs["x"], bufs["w13"], bufs["sorted_ids"], bufs["block_expert"],
                                          bufs["num_padded"], T, k, H, I, E, bm, cap, bufs["act"])


@pytest.mark.parametrize("which", ["act", "w2", "y"])
def test_down_and_combine_bindings_reject_short_buffers(which):
    T, H, E, k, I, bm = 10, 64, 8, 2, 32, 16
    cap = moe.moe_align_capacity(T, k, E, bm)
    bf = torch.bfloat16
    bufs = dict(act=_t(cap * I, bf), w2=_t(E * H * I, bf), y=_t(T * k * H, torch.float16))
    bufs[which] = _t(bufs[which].numel() - 1, bufs[which].dtype)
    with pytest.raises(ValueError, match=which):
        moe.moe_grouped_gemm_down(bufs["act"], bufs["w2"], _t(cap), _t(cap // bm), _t(1), T, k, H, I, E, bm, cap,
                                  bufs["y"])
    if which == "y":
        with pytest.raises(ValueError, match="y"):
            moe.moe_combine(bufs["y"], _t(T * k, torch.float32), T, k, H, _t(T * H, bf))
    with pytest.raises(ValueError, match="out"):
        moe.moe_combine(_t(T * k * H, torch.float16), _t(T * k, torch.float32), T, k, H, _t(T * H - 8, bf))


def test_layer_rejects_buffers_of_another_shape():
    """Buffers allocated for one (T, k, E, block_m) cannot be reused for a call
    whose capacity or shapes differ."""
    from sparse_mixture_experts_softmax_amd.layer import check_buffers

    b = moe.allocate(64, 128, 8, 2, 64, "cpu", block_m=16)
    check_buffers(b, 64, 128, 8, 2, 64, "cpu")  # the shape it was made for
    with pytest.raises(ValueError, match="cap|logits"):
        check_buffers(b, 65, 128, 8, 2, 64, "cpu")
    with pytest.raises(ValueError, match="cap"):
        check_buffers(b, 200, 128, 8, 2, 64, "cpu")
    with pytest.raises(ValueError, match="act"):
        check_buffers(b, 64, 128, 8, 2, 96, "cpu")
    with pytest.raises(ValueError, match="out|y"):
        check_buffers(b, 64, 192, 8, 2, 64, "cpu")
    with pytest.raises(ValueError, match="cap|logits"):
        check_buffers(b, 64, 128, 9, 2, 64, "cpu")


def test_binding_rejects_negative_sizes():
    with pytest.raises(ValueError, match="non-negative"):
        moe.moe_combine(_t(8, torch.float16), _t(1, torch.float32), -1, 1, 64, _t(64, torch.bfloat16))


def test_noalloc_align_validation_without_gpu():
    """The allocation-free grouping call checks its arguments on the host:
    invalid shapes and sizes beyond its static scratch are refused before any
    device work, and T = 0 succeeds."""
    L = _raw()
    args = (FAKE, FAKE, FAKE, FAKE, NULL)
    assert L.moe_align_by_expert_noalloc(FAKE, 16, 2, 8, 48, *args) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_align_by_expert_noalloc(FAKE, -1, 2, 8, 16, *args) == _lib.MOE_ERR_INVALID
    assert L.moe_align_by_expert_noalloc(FAKE, 0, 2, 8, 16, *args) == _lib.MOE_OK
    assert L.moe_align_by_expert_noalloc(NULL, 16, 2, 8, 16, *args) == _lib.MOE_ERR_INVALID
    T, k, E, bm = 300000, 8, 256, 128
    assert moe.moe_align_workspace_bytes(T, k, E, bm) > moe.moe_align_noalloc_max_workspace_bytes()
    assert L.moe_align_by_expert_noalloc(FAKE, T, k, E, bm, *args) == _lib.MOE_ERR_UNSUPPORTED
    assert "static scratch" in moe.moe_last_error()
    hdr = open(HEADER).read()
    assert f"#define MOE_ALIGN_NOALLOC_MAX_WORKSPACE_BYTES {moe.moe_align_noalloc_max_workspace_bytes()}" in hdr
