"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing ids and the expert-grouped permutation are compared bit for bit
(given the same fp32 logits); each GEMM and the combine are compared with
the oracle step they implement, fed the GPU's own upstream intermediate;
the whole layer is compared with the oracle on all five workloads within
max|err| <= 2e-2 * rms(out) + 1e-3 (and, on the tiny workload, also without
the 1e-3 floor)."""
import dataclasses
import functools
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_mixture_experts_softmax_amd as moe
from gpu_cases import (CONFIG_NAMES, act_blocks, act_rows, bf16_tensor, custom_inputs, device_inputs, host_inputs,
                       layer_tolerance, log, logits_bound, pack_reference, run_layer, sample_tokens, to_bits)

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def elem_close(gpu, ref, rel=2.0 ** -8, floor_frac=1e-3, what=""):
    """|gpu - ref| <= rel*|ref| + floor_frac*rms(ref) elementwise: bf16
    rounding of the stored result (<= 2^-9 relative) plus fp32 accumulation
    (orders of magnitude below the floor)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = rel * np.abs(ref) + floor_frac * rms
    err = np.abs(gpu - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} elements out of bound; max err {err.max():.3e}, rms {rms:.3e}"
    return float(err.max()) if err.size else 0.0


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_route_bitexact_given_logits(name):
    log(f"route {name}")
    inp = host_inputs(name)
    s = inp.shape
    dev = device_inputs(inp, key=name)
    logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    moe.moe_route(dev["x"], dev["w_router"], dev["bias"], logits, ids, w, s.T, s.H, s.E, s.k, s.norm_topk_prob)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    o_ids, o_w = oracle.select_topk(lg, s.k, s.norm_topk_prob)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    assert np.abs(w.cpu().numpy() - o_w).max() <= 1e-6
    toks = sample_tokens(s.T, 256)
    ref = oracle.router_logits(inp.x[toks], inp.w_router, inp.router_bias)
    assert (np.abs(lg[toks] - ref) <= logits_bound(inp, toks)).all()


@pytest.mark.parametrize("E,k,norm", [(8, 2, True), (128, 8, True), (128, 8, False), (256, 32, True), (5, 5, False),
                                      (1, 1, True), (256, 16, True), (200, 8, False), (129, 17, True)])
def test_route_ties_from_given_logits(E, k, norm):
    """Integer-valued logits force ties: lower expert index first. k <= 16
    takes the 16-lanes-per-token kernel (8 or 16 logits per lane), larger k
    the wave-per-token one."""
    rng = np.random.default_rng(E * 100 + k)
    T = 203
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    logits = torch.from_numpy(lg).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(None, None, None, logits, ids, w, T, 0, E, k, norm)
    torch.cuda.synchronize()
    o_ids, o_w = oracle.select_topk(lg, k, norm)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    assert np.abs(w.cpu().numpy() - o_w).max() <= 1e-6
    assert np.array_equal(logits.cpu().numpy(), lg)  # logits are input only


@pytest.mark.parametrize("T,H,E", [(333, 512, 40), (1000, 2048, 128), (300, 4096, 256), (17000, 512, 32),
                                   (8192, 512, 128), (16384, 512, 128)])
def test_router_logits_same_bits_for_small_and_large_batches(T, H, E):
    """Batches above 256 tokens take the workgroup-shared router kernel (32,
    64 or 128 experts per workgroup as the batch grows: the last two cases);
    a token's logits must not depend on which kernel (batch size) computed
    them, and both must match the oracle."""
    inp = custom_inputs(f"router{T}", T, H, E, min(8, E), 64, seed=T + H)
    dev = device_inputs(inp)

    def route(n):
        lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((n, min(8, E)), dtype=torch.int32, device="cuda")
        w = torch.empty((n, min(8, E)), dtype=torch.float32, device="cuda")
        moe.moe_route(dev["x"][:n].contiguous(), dev["w_router"], dev["bias"], lg, ids, w, n, H, E, min(8, E), True)
        torch.cuda.synchronize()
        return lg.cpu().numpy()

    big, small = route(T), route(200)
    assert np.array_equal(big[:200].view(np.uint32), small.view(np.uint32))
    toks = sample_tokens(T, 64)
    ref = oracle.router_logits(inp.x[toks], inp.w_router, inp.router_bias)
    assert (np.abs(big[toks] - ref) <= logits_bound(inp, toks)).all()


def test_route_special_logits_rank_order():
    """Signed zeros tie (lower index first), -inf can be picked, NaN ranks
    below every number and still yields a valid, distinct expert id."""
    E, k = 128, 8
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((6, E)).astype(np.float32) - 10.0
    lg[0, 5], lg[0, 1] = 0.0, -0.0                    # tie between -0 and +0
    lg[1, :] = -np.inf
    lg[1, [7, 3]] = [1.0, 2.0]                        # then -inf picks, lowest index first
    lg[2, :] = np.nan
    lg[2, [100, 9, 50]] = [-np.inf, 3.0, -1.0]        # NaN last
    lg[3, ::2] = np.nan                               # half NaN
    lg[4, :] = 0.0                                    # all tied
    lg[5, 10] = np.inf
    logits = torch.from_numpy(lg).cuda()
    ids = torch.empty((6, k), dtype=torch.int32, device="cuda")
    w = torch.empty((6, k), dtype=torch.float32, device="cuda")
    moe.moe_route(None, None, None, logits, ids, w, 6, 0, E, k, True)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(6):
        row = lg[t].astype(np.float64)
        nan = np.isnan(row)
        # rank: numbers by value (descending, -0 == +0), then NaN; ties -> lower index
        order = sorted(range(E), key=lambda e: (1, 0.0, e) if nan[e] else (0, -row[e], e))
        assert list(got[t]) == order[:k], (t, got[t], order[:k])
    assert list(got[0][:2]) == [1, 5]
    assert list(got[1][:2]) == [3, 7] and list(got[1][2:]) == [0, 1, 2, 4, 5, 6]
    assert list(got[2][:3]) == [9, 50, 100]


# ----------------------------------------------------------------------------
# Expert-grouped permutation
# ----------------------------------------------------------------------------
def _align_gpu(ids_np, E, bm, offset=0):
    """offset: pass the ids as a view that starts ``offset`` int32s into its
    allocation (offset 1: not 16-byte aligned)."""
    T, k = ids_np.shape
    cap = moe.moe_align_capacity(T, k, E, bm)
    flat = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32).reshape(-1))
    buf = torch.zeros((offset + T * k,), dtype=torch.int32, device="cuda")
    buf[offset:] = flat.cuda()
    ids = buf[offset:].view(T, k)
    sorted_ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    block_expert = torch.full((cap // bm,), -7, dtype=torch.int32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    npad = torch.empty((1,), dtype=torch.int32, device="cuda")
    wsb = moe.moe_align_workspace_bytes(T, k, E, bm)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda") if wsb else None
    moe.moe_align_by_expert(ids, T, k, E, bm, sorted_ids, block_expert, counts, npad, ws)
    torch.cuda.synchronize()
    return sorted_ids.cpu().numpy(), block_expert.cpu().numpy(), counts.cpu().numpy(), int(npad.item())


def _check_align(ids_np, E, bm, offset=0):
    g = _align_gpu(ids_np, E, bm, offset)
    o = oracle.align(ids_np, E, bm)
    assert np.array_equal(g[0], o[0]), "sorted_ids"
    assert np.array_equal(g[1], o[1]), "block_expert"
    assert np.array_equal(g[2], o[2]), "expert_counts"
    assert g[3] == o[3], "num_padded"


@pytest.mark.parametrize("name", CONFIG_NAMES)
@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_align_bitexact_on_routed_ids(name, bm):
    inp = host_inputs(name)
    s = inp.shape
    ids, _ = oracle.select_topk(oracle.router_logits(inp.x, inp.w_router, inp.router_bias), s.k) if s.T <= 64 else (
        None, None)
    if ids is None:  # large workloads: route on the GPU (bit-exact by the routing test)
        dev = device_inputs(inp, key=name)
        logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
        idt = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
        w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
        moe.moe_route(dev["x"], dev["w_router"], dev["bias"], logits, idt, w, s.T, s.H, s.E, s.k, True)
        ids = idt.cpu().numpy()
    _check_align(ids, s.E, bm)


@pytest.mark.parametrize("T,k,E,bm", [(1, 1, 1, 16), (1, 8, 128, 128), (512, 8, 128, 16), (513, 8, 128, 64),
                                      (4097, 1, 3, 32), (3000, 32, 256, 128), (777, 5, 7, 16), (20000, 2, 2, 64)])
def test_align_bitexact_edge_shapes(T, k, E, bm):
    rng = np.random.default_rng(T + k + E)
    p = rng.dirichlet(np.full(E, 0.2))
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) if np.count_nonzero(p) >= k
                    else rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _check_align(ids, E, bm)


@pytest.mark.parametrize("T,k,E,bm", [(4097, 1, 3, 32), (513, 8, 128, 64), (1024, 8, 128, 128), (1, 8, 128, 16),
                                      (4096, 8, 128, 128)])
@pytest.mark.parametrize("offset", [0, 1])
def test_align_bitexact_aligned_and_unaligned_ids(T, k, E, bm, offset):
    """Up to 8192 pairs the grouping counts all pairs inside its scatter
    kernel with 16-byte loads when the ids are 16-byte aligned, and takes
    the two-kernel path (histogram kernel + workspace) when they are not or
    when there are more pairs: all give the oracle's grouping, ragged pair
    counts included."""
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _check_align(ids, E, bm, offset)


# ----------------------------------------------------------------------------
# Weight packing
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("E,N,K,gated", [(3, 64, 64, True), (2, 96, 160, False), (5, 1536, 2048, True),
                                         (4, 2048, 768, False), (1, 32, 32, True)])
def test_pack_weights_matches_layout_definition(E, N, K, gated):
    bits = synth.normal_bf16(E * N + K, 99, (E, N, K), 1.0)
    src = bf16_tensor(bits)
    dst = torch.empty_like(src)
    moe.moe_pack_weights(src, dst, E, N, K, gated)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(dst), pack_reference(bits, gated))
    assert np.array_equal(to_bits(src), bits)  # input untouched


# ----------------------------------------------------------------------------
# Each kernel against the oracle step it implements
# ----------------------------------------------------------------------------
F16, F32 = torch.float16, torch.float32


def rows_covering_every_block(sorted_ids, npad, bm, n_pairs, seed=0):
    """Real rows of the permutation to check: all of them for small cases;
    otherwise, in every row block, the first and the last real row and one
    seeded random real row, so every (row block, column tile) of both GEMMs
    (each expert's last, partly padded block included) has checked rows."""
    real = np.nonzero(sorted_ids[:npad] != n_pairs)[0]
    if real.size <= 256:
        return real
    rng = np.random.default_rng(seed)
    pick = []
    blocks = real // bm
    starts = np.searchsorted(blocks, np.arange(npad // bm))
    ends = np.searchsorted(blocks, np.arange(npad // bm), side="right")
    for lo, hi in zip(starts, ends):
        if hi > lo:
            pick += [real[lo], real[hi - 1], real[rng.integers(lo, hi)]]
    return np.unique(np.array(pick))


@pytest.mark.parametrize("name,y_dtype", [("tiny", F16), ("tiny", F32), ("decode", F16), ("decode", F32),
                                          ("medium", F16), ("prefill", F16), ("prefill", F32), ("skewed", F16), ("skewed", F32),
                                          ("large", F16)])
def test_gemms_and_combine_against_oracle_steps(name, y_dtype):
    log(f"steps {name} y {y_dtype}")
    inp = host_inputs(name)
    s = inp.shape
    dev = device_inputs(inp, key=name)
    out, b = run_layer(inp, dev, y_dtype=y_dtype)
    assert b.y.dtype == y_dtype
    sorted_ids = b.sorted_ids.cpu().numpy()
    block_expert = b.block_expert.cpu().numpy()
    npad = int(b.num_padded.item())
    n = s.T * s.k
    rows = rows_covering_every_block(sorted_ids, npad, b.block_m, n)
    pads = np.nonzero(sorted_ids[:npad] == n)[0]
    blocks_checked = np.unique(rows // b.block_m).size
    blocks_real = np.unique(np.nonzero(sorted_ids[:npad] != n)[0] // b.block_m).size
    log(f"  {rows.size} rows checked, covering {blocks_checked} of {blocks_real} row blocks")
    assert blocks_checked == blocks_real
    act = act_rows(b.act)
    # pad rows of act are zero
    if pads.size:
        assert not _f64(act[torch.from_numpy(pads).cuda()]).any()
    x64 = synth.bf16_to_f64(inp.x)
    act_ref, act_gpu, y_ref, y_gpu = [], [], [], []
    act_sel = _f64(act[torch.from_numpy(rows).cuda()])
    y_sel = _f64(b.y[torch.from_numpy(sorted_ids[rows].astype(np.int64)).cuda()])
    for q, r in enumerate(rows):
        i = int(sorted_ids[r])
        t, e = i // s.k, int(block_expert[r // b.block_m])
        act_ref.append(oracle.expert_gate_up(x64[t], inp.w13[e])[0])
        a_gpu = act_sel[q]
        act_gpu.append(a_gpu)
        y_ref.append(oracle.expert_down(a_gpu, inp.w2[e])[0])
        y_gpu.append(y_sel[q])
    elem_close(np.array(act_gpu), np.array(act_ref), what="gate_up act")
    # fp32 accumulation error (far below the floor), plus the rounding of the
    # stored y: half an fp16 ulp (2^-11 relative; fp16 subnormals, below
    # 6.1e-5, are far below the floor)
    rel = 1e-5 + (2.0 ** -11 if y_dtype == F16 else 0.0)
    elem_close(np.array(y_gpu), np.array(y_ref), rel=rel, floor_frac=1e-4, what="down y")
    # combine, every token: fp32 output against the oracle's weighted sum of
    # the GPU's y (in chunks of tokens to bound host memory)
    out32 = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    moe.moe_combine(b.y, b.topk_weights, s.T, s.k, s.H, out32)
    torch.cuda.synchronize()
    w_all = b.topk_weights.cpu().numpy().astype(np.float64)
    for t0 in range(0, s.T, 1024):
        t1 = min(s.T, t0 + 1024)
        y3 = _f64(b.y[t0 * s.k:t1 * s.k]).reshape(t1 - t0, s.k, s.H)
        w3 = w_all[t0:t1]
        ref = oracle.combine(y3, w3)
        tol = (s.k + 1) * 2.0 ** -23 * (np.abs(w3)[:, :, None] * np.abs(y3)).sum(1) + 1e-30  # fp32 sum of k products
        assert (np.abs(_f64(out32[t0:t1]) - ref) <= tol).all(), f"combine fp32, tokens {t0}..{t1}"
        elem_close(_f64(out[t0:t1]), ref, rel=2.0 ** -8, floor_frac=1e-6, what=f"combine bf16, tokens {t0}..{t1}")


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------
@functools.lru_cache(maxsize=1)
def oracle_layer_all_tokens(name):
    """The oracle's output for every token of a workload (cached: the fp64
    per-token loop takes seconds to tens of seconds at the large shapes)."""
    inp = host_inputs(name)
    s = inp.shape
    t0 = time.perf_counter()
    ref = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob, inp.router_bias)
    log(f"  oracle: {s.T} tokens of {name} in {time.perf_counter() - t0:.1f} s "
        f"({oracle.default().max_threads()} threads)")
    return ref


def bf16_rne(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of finite fp32 values, round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |ref| (the rounding error of a
    correctly rounded bf16 result): 2^(floor(log2|ref|) - 8)."""
    a = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 8)


@pytest.mark.parametrize("name,y_dtype", [("tiny", F16), ("tiny", F32), ("decode", F16), ("medium", F16),
                                          ("prefill", F16), ("skewed", F16), ("large", F16), ("large", F32)])
def test_layer_matches_oracle(name, y_dtype):
    """Every token of every workload (so every row block and column tile of
    both GEMMs) against the oracle.

    The tolerance max|err| <= 2e-2 * rms(out) + 1e-3 is stated for the layer
    with bf16 inputs and fp32 accumulation: it holds the layer's fp32 result
    (out_dtype fp32). The bf16 output must then be exactly that fp32 result
    rounded to nearest even, and within the bound plus the half bf16 ulp any
    bf16-typed result carries (at the large workload the biggest outputs
    exceed 2, where that half ulp, 2^-7, is above the bound itself)."""
    log(f"layer {name} y {y_dtype}")
    inp = host_inputs(name)
    s = inp.shape
    dev = device_inputs(inp, key=name)
    out32, b = run_layer(inp, dev, y_dtype=y_dtype, out_dtype=torch.float32)
    out16, b16 = run_layer(inp, dev, y_dtype=y_dtype)
    ref, ref_ids, ref_w = oracle_layer_all_tokens(name)
    got = _f64(out32)
    assert got.shape == ref.shape
    assert np.isfinite(got).all()
    assert np.array_equal(b.topk_ids.cpu().numpy(), ref_ids)
    assert np.abs(b.topk_weights.cpu().numpy() - ref_w).max() <= 1e-6
    err = np.abs(got - ref).max()
    tol = layer_tolerance(ref)
    rms = np.sqrt(np.mean(ref ** 2))
    log(f"  {name}: fp32 output max err {err:.3e}, bound {tol:.3e}, rms {rms:.3e}, max|out| {np.abs(ref).max():.3f}")
    assert err <= tol
    if name == "tiny":
        assert err <= layer_tolerance(ref, floor=False)
    # the bf16 output is the fp32 result rounded to nearest even
    assert np.array_equal(to_bits(out16), bf16_rne(out32.cpu().numpy()))
    err16 = np.abs(_f64(out16) - ref)
    log(f"  {name}: bf16 output max err {err16.max():.3e}")
    assert (err16 <= tol + bf16_half_ulp(ref)).all()


def test_layer_edge_cases():
    cases = [
        ("one_token", 1, 256, 16, 4, 64, True),
        ("ragged", 37, 128, 8, 2, 96, True),
        ("dense", 45, 128, 1, 1, 64, True),
        ("k_eq_E", 20, 64, 8, 8, 32, False),
        ("wide", 33, 1024, 256, 32, 32, True),
        ("no_renorm", 50, 192, 12, 3, 160, False),
        ("multi_tile", 600, 64, 16, 8, 64, True),
        # 128-row blocks through the pipelined wide kernel with ragged N
        # tiles (I and H below one tile) and an odd k-step count (I/32 = 5)
        ("wide_ragged", 700, 192, 8, 2, 160, True),
        ("wide_odd", 520, 128, 4, 1, 96, False),
    ]
    for name, T, H, E, k, I, norm in cases:
        log(f"edge {name}")
        inp = custom_inputs(name, T, H, E, k, I, norm=norm, seed=T)
        out, b = run_layer(inp)
        ref, ref_ids, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, k, norm)
        assert np.array_equal(b.topk_ids.cpu().numpy(), ref_ids), name
        err = np.abs(_f64(out) - ref).max()
        assert err <= layer_tolerance(ref), (name, err)


def test_zero_tokens_is_a_noop():
    """T = 0: every entry point returns success and writes nothing. Each call
    gets real, sentinel-filled buffers (sized for T = 4) and they must come
    back unchanged; the layer returns an empty [0, H] output."""
    inp = custom_inputs("empty", 4, 64, 8, 2, 32)
    dev = device_inputs(inp)
    b = moe.allocate(4, 64, 8, 2, 32, "cuda", block_m=16)
    for name in ("logits", "topk_weights", "act", "y", "out"):
        getattr(b, name).fill_(3.0)
    for name in ("topk_ids", "sorted_ids", "block_expert", "expert_counts", "num_padded"):
        getattr(b, name).fill_(-5)
    before = {f.name: getattr(b, f.name).clone() for f in dataclasses.fields(b)
              if isinstance(getattr(b, f.name), torch.Tensor)}
    x, pk = dev["x"], dev["packed"]
    moe.moe_route(x, dev["w_router"], None, b.logits, b.topk_ids, b.topk_weights, 0, 64, 8, 2, True)
    moe.moe_route(None, None, None, b.logits, b.topk_ids, b.topk_weights, 0, 0, 8, 2, True)
    moe.moe_align_by_expert(b.topk_ids, 0, 2, 8, 16, b.sorted_ids, b.block_expert, b.expert_counts, b.num_padded)
    moe.moe_grouped_gemm_gate_up_silu(x, pk.w13, b.sorted_ids, b.block_expert, b.num_padded, 0, 2, 64, 32, 8, 16,
                                      0, b.act)
    moe.moe_grouped_gemm_down(b.act, pk.w2, b.sorted_ids, b.block_expert, b.num_padded, 0, 2, 64, 32, 8, 16, 0, b.y)
    moe.moe_combine(b.y, b.topk_weights, 0, 2, 64, b.out)
    torch.cuda.synchronize()
    for name, t in before.items():
        assert torch.equal(getattr(b, name), t), f"{name} was written by a T = 0 call"
    res = moe.moe_layer(x[:0], dev["w_router"], top_k=2, packed=pk)
    torch.cuda.synchronize()
    assert res.shape == (0, 64) and res.dtype == torch.bfloat16 and res.device == x.device


@pytest.mark.parametrize("bm", [16, 32, 128])
def test_expert_outputs_beyond_fp16_range(bm):
    """Expert outputs far beyond +-65504 (the down weights scaled by 2^23,
    exact in bf16). With fp32 y the layer still matches the oracle; with fp16
    y an output element is non-finite exactly where one of its token's k
    expert outputs rounds past the fp16 range (|y| >= 65520, judged on the
    fp32 y of the same run), and finite and unchanged elsewhere."""
    base = custom_inputs(f"bigy{bm}", 160, 256, 8, 2, 128, seed=21)
    s = base.shape
    w2 = (synth.bf16_to_f64(base.w2) * 2.0 ** 23).astype(np.float32)
    w2_bits = (w2.view(np.uint32) >> 16).astype(np.uint16)  # exact: a power-of-two scale of bf16 values
    inp = synth.MoEInputs(s, base.seed, base.x, base.w_router, base.w13, w2_bits, None)
    o32, b32 = run_layer(inp, block_m=bm, y_dtype=F32)
    o16, b16 = run_layer(inp, block_m=bm, y_dtype=F16)
    ref, _, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob)
    y32 = _f64(b32.y).reshape(s.T, s.k, s.H)
    assert np.abs(y32).max() > 1e5  # the case is real
    got32 = _f64(o32)
    assert np.isfinite(got32).all()
    assert np.abs(got32 - ref).max() <= layer_tolerance(ref)
    over = (np.abs(y32) >= 65520.0).any(axis=1)
    got16 = _f64(o16)
    assert np.array_equal(~np.isfinite(got16), over)
    assert over.any() and (~over).any()
    fin = ~over
    assert np.abs(got16[fin] - ref[fin]).max() <= layer_tolerance(ref)


# ----------------------------------------------------------------------------
# Structure: poisoning, determinism, batch split, relabelling, tile size
# ----------------------------------------------------------------------------
def test_nan_poison_unused_experts_and_pad_rows():
    inp = custom_inputs("poison", 300, 256, 32, 4, 128, skewed=True, seed=3)
    s = inp.shape
    clean, bc = run_layer(inp, block_m=32)
    counts = bc.expert_counts.cpu().numpy()
    unused = np.nonzero(counts == 0)[0]
    assert unused.size >= 5
    w13p, w2p = inp.w13.copy(), inp.w2.copy()
    w13p[unused] = NAN_BF16
    w2p[unused] = NAN_BF16
    dev = device_inputs(inp)
    dev = dict(dev, w13=bf16_tensor(w13p), w2=bf16_tensor(w2p))
    dev["packed"] = moe.pack_experts(dev["w13"], dev["w2"])
    out, b = run_layer(inp, dev, block_m=32)
    assert np.array_equal(to_bits(out), to_bits(clean))
    # poison pad rows of act between the two GEMMs
    n = s.T * s.k
    pad = torch.from_numpy(np.nonzero(b.sorted_ids.cpu().numpy() == n)[0]).cuda()
    rows = act_rows(b.act).clone()
    rows[pad] = float("nan")
    b.act.copy_(act_blocks(rows))
    moe.moe_grouped_gemm_down(b.act, dev["packed"].w2, b.sorted_ids, b.block_expert, b.num_padded, s.T, s.k, s.H,
                              s.I, s.E, b.block_m, b.cap, b.y)
    out2 = torch.empty_like(out)
    moe.moe_combine(b.y, b.topk_weights, s.T, s.k, s.H, out2)
    torch.cuda.synchronize()
    assert torch.isfinite(out2.float()).all()
    assert np.array_equal(to_bits(out2), to_bits(clean))


@pytest.mark.parametrize("name", ["decode", "medium", "prefill", "skewed", "large"])
def test_run_twice_bit_identical(name):
    inp = host_inputs(name)
    dev = device_inputs(inp, key=name)
    o1, b1 = run_layer(inp, dev)
    o2, b2 = run_layer(inp, dev)
    for f in ("topk_ids", "sorted_ids", "block_expert", "expert_counts", "num_padded"):
        assert torch.equal(getattr(b1, f), getattr(b2, f)), f
    for f in ("logits", "topk_weights"):
        assert torch.equal(getattr(b1, f), getattr(b2, f)), f
    npad = int(b1.num_padded.item())
    assert np.array_equal(to_bits(b1.act[:npad]), to_bits(b2.act[:npad]))
    assert np.array_equal(to_bits(b1.y), to_bits(b2.y))
    assert np.array_equal(to_bits(o1), to_bits(o2))


@pytest.mark.parametrize("bm", [64, 128])
def test_batch_split_bit_identical(bm):
    inp = host_inputs("prefill")
    s = inp.shape
    dev = device_inputs(inp, key="prefill")
    full, _ = run_layer(inp, dev, block_m=bm)
    half = s.T // 2
    sub = synth.MoEInputs(s.with_tokens(half), 0, inp.x[:half], inp.w_router, inp.w13, inp.w2, inp.router_bias)
    dsub = dict(dev, x=dev["x"][:half].contiguous())
    part, _ = run_layer(sub, dsub, block_m=bm)
    assert np.array_equal(to_bits(part), to_bits(full[:half]))


def test_expert_relabelling_bit_identical():
    inp = custom_inputs("relabel", 700, 256, 24, 4, 128, seed=5)
    out, _ = run_layer(inp, block_m=16)
    perm = np.random.default_rng(2).permutation(24)
    p = synth.MoEInputs(inp.shape, 5, inp.x, inp.w_router[perm], inp.w13[perm], inp.w2[perm], None)
    out_p, _ = run_layer(p, block_m=16)
    assert np.array_equal(to_bits(out_p), to_bits(out))


def test_block_m_changes_results_only_by_rounding():
    """16/32 and 64/128/256 share an MFMA shape: bit-identical within each
    group (256-row blocks run as two 128-row tiles); across shapes the fp32
    accumulation order differs, so outputs agree to bf16 rounding and each
    matches the oracle."""
    inp = custom_inputs("tiles", 900, 512, 16, 4, 256, seed=9)
    outs = {bm: run_layer(inp, block_m=bm)[0] for bm in (16, 32, 64, 128, 256)}
    assert np.array_equal(to_bits(outs[16]), to_bits(outs[32]))
    assert np.array_equal(to_bits(outs[64]), to_bits(outs[128]))
    assert np.array_equal(to_bits(outs[128]), to_bits(outs[256]))
    a, b = _f64(outs[16]), _f64(outs[64])
    assert (np.abs(a - b) <= 2.0 ** -7 * np.abs(a) + 1e-3 * np.sqrt(np.mean(a ** 2))).all()
    ref, _, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 4, True)
    for bm, o in outs.items():
        assert np.abs(_f64(o) - ref).max() <= layer_tolerance(ref), bm


@pytest.mark.parametrize("T", [40, 150, 600])
def test_single_and_shared_expert_blocks(T):
    """Row blocks that are their expert's only one load the weights with a
    different cache policy from blocks that share an expert: T = 40 gives
    every expert one 16- or 32-row block, 150 a mix, 600 several per expert.
    Same values either way: 16- and 32-row blocks agree bit for bit, and
    both match the oracle."""
    inp = custom_inputs(f"blocks{T}", T, 256, 16, 4, 128, seed=T)
    outs = {bm: run_layer(inp, block_m=bm)[0] for bm in (16, 32)}
    assert np.array_equal(to_bits(outs[16]), to_bits(outs[32]))
    ref, _, _ = oracle.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 4, True)
    assert np.abs(_f64(outs[16]) - ref).max() <= layer_tolerance(ref)


def test_python_errors_on_gpu():
    inp = custom_inputs("err", 8, 64, 8, 2, 32)
    dev = device_inputs(inp)
    with pytest.raises(moe.MoEError, match="k="):
        moe.moe_layer(dev["x"], dev["w_router"], top_k=9, packed=dev["packed"])
    with pytest.raises(ValueError, match="shape mismatch"):
        moe.moe_layer(dev["x"], dev["w_router"], dev["w2"], dev["w2"], top_k=2)
    # row-major weights are packed on the fly and give the same result
    a = moe.moe_layer(dev["x"], dev["w_router"], dev["w13"], dev["w2"], top_k=2)
    b = moe.moe_layer(dev["x"], dev["w_router"], top_k=2, packed=dev["packed"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
