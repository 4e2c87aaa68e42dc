"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError when
the oracle disagrees with an independent fact: a hand-worked closed-form
example, a brute-force formulation that evaluates every expert for every
token, the PyTorch CPU routines the pages name (F.linear, softmax,
torch.topk, F.silu) in float64, closed forms of the routing weights, and the
invariants of the layer and of the expert-grouped permutation. The battery is
run against the real oracle and against mutated copies of it (each must fail
at least one pin).
"""
from __future__ import annotations

import functools
import json
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
REL = 1e-12  # agreement of two float64 formulations of the same definition


def bf16_bits(values) -> np.ndarray:
    """float values that are exactly representable in bf16 -> bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(synth.bf16_to_f64(bits), f.astype(np.float64)), "value not exact in bf16"
    return bits


def _close(a, b, rel=REL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.abs(b).max(initial=0.0)))
    err = float(np.abs(a - b).max(initial=0.0))
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:.1e} * {scale:.3e}"


@functools.lru_cache(maxsize=None)
def small_inputs(name, T, H, E, k, I, norm=True, skewed=False, seed=0):
    shape = synth.MoEShape(name, T, H, E, k, I, norm_topk_prob=norm, skewed=skewed)
    return synth.make_inputs(shape, seed=seed)


@functools.lru_cache(maxsize=None)
def config_inputs(name, seed=0):
    return synth.make_inputs(synth.CONFIGS[name], seed=seed)


# ----------------------------------------------------------------------------
# Hand-worked example
# ----------------------------------------------------------------------------
def pin_worked_example(orc):
    fx = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    x, wr = bf16_bits(fx["x"]), bf16_bits(fx["w_router"])
    w13, w2 = bf16_bits(fx["w13"]), bf16_bits(fx["w2"])
    for case in fx["cases"]:
        out, ids, w = orc.moe_layer(x, wr, w13, w2, fx["k"], norm_topk_prob=case["norm_topk_prob"])
        assert ids.tolist() == case["ids"], (ids, case["ids"])
        _close(w, case["weights"], 1e-14, "worked example weights")
        _close(out, case["out"], 1e-14, "worked example output")
    tie = fx["tie_case"]
    ids, w = orc.select_topk(np.array(tie["logits"]), tie["k"], True)
    assert ids.tolist() == tie["ids"]
    _close(w, tie["weights_renorm"], 1e-15, "tie renorm")
    ids, w = orc.select_topk(np.array(tie["logits"]), tie["k"], False)
    assert ids.tolist() == tie["ids"]
    _close(w, tie["weights_plain"], 1e-15, "tie plain")


def pin_printed_shapes(orc):
    """The page prints the merged gate_up weight as [2I, H] and the down
    weight as [H, I]; the oracle's expert MLP takes exactly those shapes."""
    fx = json.load(open(os.path.join(GOLDEN, "printed_shapes.json")))
    H, I = fx["hidden_size"], fx["intermediate_size"]
    shape = synth.MoEShape("printed", 1, H, 1, 1, I)
    w13, w2 = synth.expert_weights(shape, seed=0)
    assert list(w13.shape[1:]) == fx["gate_up_proj"] and list(w2.shape[1:]) == fx["down_proj"]
    x = np.zeros((1, H))
    x[0, 0] = 1.0
    y = orc.expert_mlp(x, w13[0], w2[0])
    assert y.shape == (1, H)


# ----------------------------------------------------------------------------
# Brute force: every expert for every token, dense combine matrix
# ----------------------------------------------------------------------------
def dense_reference(inp, k, norm):
    """Evaluates ALL experts for every token and combines them with a dense
    [T, E] matrix that is zero off each token's k best experts. Selection is
    by brute-force rank: expert e is chosen iff fewer than k experts rank
    before it (larger logit, or equal logit and lower index)."""
    x = synth.bf16_to_f64(inp.x)
    wr = synth.bf16_to_f64(inp.w_router)
    w13 = synth.bf16_to_f64(inp.w13)
    w2 = synth.bf16_to_f64(inp.w2)
    T, E, I = x.shape[0], wr.shape[0], w2.shape[2]
    logits = x @ wr.T
    if inp.router_bias is not None:
        logits = logits + inp.router_bias.astype(np.float64)
    p = scipy.special.softmax(logits, axis=1)
    idx = np.arange(E)
    le, lo = logits[:, :, None], logits[:, None, :]  # [t, e, e']
    before = (lo > le) | ((lo == le) & (idx[None, None, :] < idx[None, :, None]))
    rank = before.sum(axis=2)
    sel = rank < k
    G = np.where(sel, p, 0.0)
    if norm:
        G = G / G.sum(axis=1, keepdims=True)
    out = np.zeros_like(x)
    for e in range(E):
        g = x @ w13[e, :I].T
        u = x @ w13[e, I:].T
        a = g * scipy.special.expit(g) * u
        out += G[:, e:e + 1] * (a @ w2[e].T)
    ids = np.argsort(rank, axis=1, kind="stable")[:, :k]
    return out, ids, np.take_along_axis(G, ids, axis=1), logits


def pin_bruteforce(orc):
    cases = [
        (config_inputs("tiny"), 2, True),
        (small_inputs("s1", 37, 96, 12, 3, 40, norm=False), 3, False),
        (small_inputs("s2", 29, 128, 16, 4, 64, skewed=True), 4, True),
        (small_inputs("s3", 9, 64, 5, 5, 32, norm=False, seed=3), 5, False),
    ]
    for inp, k, norm in cases:
        out, ids, w = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, k, norm, inp.router_bias)
        d_out, d_ids, d_w, d_logits = dense_reference(inp, k, norm)
        _close(orc.router_logits(inp.x, inp.w_router, inp.router_bias), d_logits, REL, "logits")
        assert np.array_equal(ids, d_ids), "top-k ids differ from brute force"
        _close(w, d_w, REL, "routing weights")
        _close(out, d_out, REL, "layer output")


# ----------------------------------------------------------------------------
# The PyTorch CPU routines the pages name, in float64
# ----------------------------------------------------------------------------
def torch_reference(inp, k, norm, tokens):
    x = torch.from_numpy(synth.bf16_to_f64(inp.x[tokens]))
    wr = torch.from_numpy(synth.bf16_to_f64(inp.w_router))
    b = None if inp.router_bias is None else torch.from_numpy(inp.router_bias.astype(np.float64))
    logits = F.linear(x, wr, b)
    scores = torch.softmax(logits, dim=-1)
    w, ids = torch.topk(scores, k, dim=-1)
    if norm:
        w = w / w.sum(dim=-1, keepdim=True)
    I = inp.w2.shape[2]
    out = torch.zeros_like(x)
    for e in torch.unique(ids).tolist():
        w13 = torch.from_numpy(synth.bf16_to_f64(inp.w13[e]))
        w2 = torch.from_numpy(synth.bf16_to_f64(inp.w2[e]))
        rows, slots = torch.nonzero(ids == e, as_tuple=True)
        gu = F.linear(x[rows], w13)
        y = F.linear(F.silu(gu[:, :I]) * gu[:, I:], w2)
        out.index_add_(0, rows, w[rows, slots, None] * y)
    return out.numpy(), ids.numpy(), w.numpy()


def pin_torch_library(orc):
    cases = [
        (config_inputs("tiny"), 2, True, None),
        (small_inputs("s4", 23, 192, 24, 6, 96, norm=False, seed=7), 6, False, None),
        (config_inputs("decode"), 8, True, np.array([0, 5, 17, 63])),
    ]
    for inp, k, norm, tokens in cases:
        if tokens is None:
            tokens = np.arange(inp.x.shape[0])
        out, ids, w = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, k, norm, inp.router_bias, tokens)
        t_out, t_ids, t_w = torch_reference(inp, k, norm, tokens)
        assert np.array_equal(ids, t_ids), "top-k ids differ from torch.topk"
        _close(w, t_w, REL, "weights vs torch")
        _close(out, t_out, 1e-11, "output vs torch")


# ----------------------------------------------------------------------------
# Closed forms and properties of the routing weights
# ----------------------------------------------------------------------------
def pin_weight_closed_forms(orc):
    # two experts whose logits differ by ln 3: scores 3/4 and 1/4
    ids, w = orc.select_topk(np.array([[np.log(3.0), 0.0]]), 2, False)
    assert ids.tolist() == [[0, 1]]
    _close(w, [[0.75, 0.25]], 1e-15, "ln3 pair")
    ids, w = orc.select_topk(np.array([[0.0, np.log(3.0)]]), 1, False)
    assert ids.tolist() == [[1]]
    _close(w, [[0.75]], 1e-15, "ln3 top-1")
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((50, 20)) * 2
    for k in (1, 3, 7, 20):
        ids, w = orc.select_topk(lg, k, True)
        # renormalised weights are the softmax of the selected logits alone
        sel = np.take_along_axis(lg, ids, axis=1)
        _close(w, scipy.special.softmax(sel, axis=1), 1e-14, "renorm = softmax over selected")
        _close(w.sum(1), np.ones(50), 1e-14, "sum to one")
        assert (np.diff(w, axis=1) <= 0).all(), "weights not non-increasing"
        ids_p, w_p = orc.select_topk(lg, k, False)
        assert np.array_equal(ids, ids_p)
        assert (w_p.sum(1) <= 1 + 1e-14).all()
        # unnormalised weights are the full softmax at the selected experts
        _close(w_p, np.take_along_axis(scipy.special.softmax(lg, axis=1), ids, axis=1), 1e-14, "plain")
    _close(orc.select_topk(lg, 20, False)[1].sum(1), np.ones(50), 1e-14, "k = E sums to one")


def pin_topk_bruteforce(orc):
    """Integer-valued logits force many ties; ids must follow (value desc,
    index asc), computed by Python's sort."""
    rng = np.random.default_rng(5)
    for E, k in ((8, 2), (33, 5), (128, 8), (256, 32)):
        lg = rng.integers(-3, 4, size=(40, E)).astype(np.float64)
        ids, _ = orc.select_topk(lg, k, True)
        for t in range(40):
            want = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
            assert ids[t].tolist() == want, (E, k, t)


# ----------------------------------------------------------------------------
# Expert-grouped permutation
# ----------------------------------------------------------------------------
def check_permutation(ids, E, block_m, sorted_ids, block_expert, counts, num_padded):
    """Invariants plus brute force (np.lexsort by (expert, flat index))."""
    T, k = ids.shape
    n = T * k
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E)), "counts"
    assert counts.sum() == n
    padded = (counts + block_m - 1) // block_m * block_m
    assert num_padded == padded.sum()
    real = sorted_ids[sorted_ids != n]
    # every flat index exactly once => every token exactly k times
    assert np.array_equal(np.sort(real), np.arange(n)), "not a permutation"
    assert np.array_equal(np.bincount(real // k, minlength=T), np.full(T, k))
    order = np.lexsort((np.arange(n), flat))  # by expert, then flat index
    off = 0
    for e in range(E):
        seg = sorted_ids[off:off + padded[e]]
        assert np.array_equal(seg[:counts[e]], order[off - (padded[:e] - counts[:e]).sum():][:counts[e]]), e
        assert (seg[counts[e]:] == n).all(), "pad rows must hold the sentinel"
        assert (block_expert[off // block_m:(off + padded[e]) // block_m] == e).all()
        off += padded[e]
    assert (sorted_ids[num_padded:] == n).all()
    assert (block_expert[num_padded // block_m:] == -1).all()
    assert len(padded[padded > 0]) == len(set(block_expert[block_expert >= 0].tolist())), "empty expert owns a block"


def pin_align(orc):
    rng = np.random.default_rng(2)
    for T, k, E, bm in ((16, 2, 8, 16), (64, 8, 128, 16), (500, 4, 37, 32), (300, 8, 128, 64),
                        (1000, 2, 4, 128), (7, 3, 256, 256), (1, 1, 1, 16)):
        # skewed draws leave some experts empty; rows hold distinct experts
        p = rng.dirichlet(np.full(E, 0.3))
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) if np.count_nonzero(p) >= k
                        else rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        sorted_ids, block_expert, counts, npad = orc.align(ids, E, bm)
        check_permutation(ids, E, bm, sorted_ids, block_expert, counts, npad)


# ----------------------------------------------------------------------------
# Special cases and symmetries of the layer
# ----------------------------------------------------------------------------
def pin_single_expert_is_dense_mlp(orc):
    """E = 1, k = 1: weight 1 and the layer is the dense SwiGLU GatedMLP,
    evaluated with torch.nn.functional in float64."""
    inp = small_inputs("dense", 13, 64, 1, 1, 48, seed=4)
    out, ids, w = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 1, True)
    assert (ids == 0).all() and np.all(w == 1.0)
    x = torch.from_numpy(synth.bf16_to_f64(inp.x))
    gu = F.linear(x, torch.from_numpy(synth.bf16_to_f64(inp.w13[0])))
    y = F.linear(F.silu(gu[:, :48]) * gu[:, 48:], torch.from_numpy(synth.bf16_to_f64(inp.w2[0])))
    _close(out, y.numpy(), 1e-12, "dense GatedMLP")
    for norm in (True, False):  # one expert: its score is 1 either way
        o2, _, w2 = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 1, norm)
        assert np.all(w2 == 1.0)


def pin_identical_experts(orc):
    """All experts equal: under renormalisation (any k), or with k = E and no
    renormalisation, the layer equals one expert's output."""
    inp = small_inputs("same", 11, 64, 6, 3, 32, seed=9)
    w13 = np.repeat(inp.w13[2:3], 6, axis=0)
    w2 = np.repeat(inp.w2[2:3], 6, axis=0)
    one = orc.expert_mlp(synth.bf16_to_f64(inp.x), w13[0], w2[0])
    for k, norm in ((3, True), (1, True), (6, False), (6, True)):
        out, _, _ = orc.moe_layer(inp.x, inp.w_router, w13, w2, k, norm)
        _close(out, one, 1e-13, f"identical experts k={k}")


def pin_linearity(orc):
    """Scaling the down weights by a power of two scales the output exactly."""
    inp = small_inputs("lin", 10, 64, 8, 2, 32, seed=12)
    out, _, _ = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 2, True)
    w2x2 = (inp.w2.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1 (no zeros/denormals)
    assert np.array_equal(synth.bf16_to_f64(w2x2), 2 * synth.bf16_to_f64(inp.w2))
    out2, _, _ = orc.moe_layer(inp.x, inp.w_router, inp.w13, w2x2, 2, True)
    assert np.array_equal(out2, 2 * out)


def pin_relabel(orc):
    """Permuting experts (router rows and weights together) relabels ids and
    leaves the output unchanged."""
    inp = small_inputs("relabel", 21, 64, 10, 3, 32, seed=6, skewed=True)
    perm = np.random.default_rng(1).permutation(10)
    out, ids, w = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 3, True, inp.router_bias)
    out_p, ids_p, w_p = orc.moe_layer(inp.x, inp.w_router[perm], inp.w13[perm], inp.w2[perm], 3, True,
                                      inp.router_bias[perm])
    assert np.array_equal(perm[ids_p], ids)
    _close(w_p, w, 1e-13, "relabel weights")
    _close(out_p, out, 1e-13, "relabel output")


def pin_token_subset(orc):
    """Tokens are independent: any subset of tokens gives the same rows."""
    inp = small_inputs("subset", 40, 64, 8, 2, 32, seed=8)
    out, ids, w = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 2, True)
    sub = np.array([39, 0, 17, 17, 5])
    o2, i2, w2 = orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, 2, True, tokens=sub)
    assert np.array_equal(o2, out[sub]) and np.array_equal(i2, ids[sub]) and np.array_equal(w2, w[sub])


# ----------------------------------------------------------------------------
# Fused residual add + RMSNorm (the step before the layer)
# ----------------------------------------------------------------------------
def pin_rmsnorm_worked_example(orc):
    fx = json.load(open(os.path.join(GOLDEN, "rmsnorm_worked_example.json")))
    for case in fx["cases"]:
        x = bf16_bits(case["x"])
        r = None if case["residual"] is None else bf16_bits(case["residual"])
        out, res = orc.fused_add_rmsnorm(x, r, bf16_bits(case["weight"]), fx["eps"])
        assert synth.bf16_to_f64(out).tolist() == case["out"], (case["derivation"], synth.bf16_to_f64(out))
        assert synth.bf16_to_f64(res).tolist() == case["new_residual"]


def pin_rmsnorm_library(orc):
    """torch.nn.functional.rms_norm (float64) on the new residual, times the
    weight, agrees with the oracle to within the two bf16 roundings."""
    for T, H, scale in ((7, 64, 1.0), (5, 2048, 3.0), (3, 96, 1e-4)):
        x = synth.normal_bf16(T * H, 77, (T, H), scale)
        r = synth.normal_bf16(T * H, 78, (T, H), scale)
        w = synth.normal_bf16(H, 79, (H,), 1.0)
        out, res = orc.fused_add_rmsnorm(x, r, w, 1e-6)
        r64 = torch.from_numpy(synth.bf16_to_f64(res))
        n = F.rms_norm(r64, (H,), eps=1e-6)
        ref = (n * torch.from_numpy(synth.bf16_to_f64(w))).numpy()
        got = synth.bf16_to_f64(out)
        assert (np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30).all()
        # the residual is the bf16 rounding of the fp32 sum
        s32 = (synth.bf16_to_f64(x).astype(np.float32) + synth.bf16_to_f64(r).astype(np.float32))
        ref_r = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
        assert np.array_equal(synth.bf16_to_f64(res), ref_r)


def pin_rmsnorm_closed_forms(orc):
    H = 64
    w = bf16_bits(np.ones(H))
    # constant rows: n = c / sqrt(c^2 + eps)
    for c, want in ((1.0, 1.0), (-2.0, -1.0), (2.0 ** -12, None)):
        out, res = orc.fused_add_rmsnorm(bf16_bits(np.full((1, H), c)), None, w, 1e-6)
        got = synth.bf16_to_f64(out)[0]
        if want is None:  # eps dominates: 2^-12 / sqrt(2^-24 + 1e-6)
            want = float(torch.tensor(2.0 ** -12 / np.sqrt(2.0 ** -24 + 1e-6)).to(torch.bfloat16))
        assert (got == want).all(), (c, got[0], want)
        assert np.array_equal(res, bf16_bits(np.full((1, H), c)))
    # scaling x by a power of two leaves the normalized output unchanged (eps aside)
    x = synth.normal_bf16(5, 80, (4, H), 1.0)
    a, _ = orc.fused_add_rmsnorm(x, None, w, 0.0)
    b, _ = orc.fused_add_rmsnorm((x.astype(np.uint32) + (3 << 7)).astype(np.uint16), None, w, 0.0)
    assert np.array_equal(a, b)


ALL_PINS = [
    pin_worked_example,
    pin_printed_shapes,
    pin_bruteforce,
    pin_torch_library,
    pin_weight_closed_forms,
    pin_topk_bruteforce,
    pin_align,
    pin_single_expert_is_dense_mlp,
    pin_identical_experts,
    pin_linearity,
    pin_relabel,
    pin_token_subset,
    pin_rmsnorm_worked_example,
    pin_rmsnorm_library,
    pin_rmsnorm_closed_forms,
]
