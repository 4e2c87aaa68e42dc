#!/usr/bin/env python3
"""Throughput of the fused sparse MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                    [--also medium,prefill,skewed,large] [--cpu-seconds 12]

A step is one pass of the whole layer (route, align, gate/up GEMM + SiLU*mul,
down GEMM, combine: the five C-ABI calls) over one batch of synthetic
inputs already resident in HBM (expert weights packed once, at load time).
W untimed steps, then exactly K timed steps between two device
synchronisations, with nothing else on the stream; the weights are rotated
over resident copies so the 256 MB Infinity Cache cannot serve one step's
weights to the next. That region gives ``ms_per_step`` and ``value``.

Event markers cost several microseconds each on this stream, so they stay
out of that region. A second region runs the same K steps with HIP events
recorded on the launch stream around each step and around the two GEMMs:
it gives the per-step median and p10/p90 and the GEMMs' average launch
durations, from which the roofline entry is computed (the kernel's
algorithmic bytes or flops per launch over that duration). A third, short
region with events around every call gives the per-kernel breakdown.

The headline workload (default: decode, HBM-bound) is the JSON line's
``value``; the workloads named by ``--also`` (default: the mid-batch layer,
HBM-bound like decode, and the matrix-core-bound prefill, skewed and large
layers) are measured in the same process, the same way, and reported under
``workloads``. Counter figures (HBM bytes, MFMA busy)
come from committed rocprofv3 runs (profiles/counters.json) and are reported
only while the kernel's source is unchanged since they were taken. The CPU
oracle is timed on a bounded sample of the headline workload on the host
cores (cpu_baseline), and on one core.

    python bench.py --record-counters DIR --workload W

turns the CSV output of the rocprofv3 counter passes listed in
``counter_commands(W)`` (run with ``-d DIR``) into profiles/counters.json
entries and a summary table under profiles/.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/s; achieved HBM GB/s (decode) and MFMA TFLOP/s (prefill)"
WORKLOAD_TEXT = {
    "tiny": "tiny MoE layer",
    "decode": "decode-shaped Qwen3-MoE layer",
    "prefill": "prefill-shaped Qwen3-MoE layer",
    "skewed": "skewed-routing (Zipf 1.2) MoE layer",
    "large": "large MoE layer on one GPU",
    "medium": "mid-batch Qwen3-MoE layer (512 tokens, 32 rows per expert)",
    "dense": "dense SwiGLU GatedMLP (Qwen3-0.6B MLP shape) through the grouped GEMMs",
    "add_rmsnorm": "fused residual add + RMSNorm before the layer (prefill-shaped hidden state)",
}
NORM_SHAPE = (4096, 2048)  # tokens, hidden (the prefill-shaped layer's input)
KERNELS = ["route", "align", "gate_up", "down", "combine"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = {
    "gate_up": ["gemm.hip", "moe_common.h"],
    "down": ["gemm.hip", "moe_common.h"],
    "pack": ["pack.hip"],
    "route": ["route.hip", "moe_common.h"],
    "align": ["align.hip"],
    "combine": ["combine.hip", "moe_common.h"],
}


def progress(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_mixture_experts_softmax_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_record(workload: str, kernel: str):
    """The committed counter record of one kernel on one workload, or None
    when absent or taken on a different version of the kernel's source."""
    try:
        with open(COUNTERS_FILE) as fh:
            rec = json.load(fh).get(f"{workload}/{kernel}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_hash(kernel):
        return None
    return rec


def algorithmic_work(shape, counts, y_bytes=2):
    """Per-kernel algorithmic bytes and flops for one step (each touched
    expert's weights read once; activations, router weights and outputs read
    or written once; padding, re-reads and intermediates' round trips are
    not counted). ``y_bytes``: bytes per element of the stored y."""
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I
    touched = int((counts > 0).sum())
    pairs = T * k
    b = 2  # bf16
    return {
        "route": {"bytes": T * H * b + E * H * b + T * E * 4 + pairs * 8, "flops": 2 * T * H * E},
        "align": {"bytes": pairs * 4 * 2, "flops": 0},
        "gate_up": {"bytes": touched * 2 * I * H * b + T * H * b + pairs * I * b, "flops": 2 * pairs * 2 * I * H},
        "down": {"bytes": touched * H * I * b + pairs * I * b + pairs * H * y_bytes, "flops": 2 * pairs * H * I},
        "combine": {"bytes": pairs * H * y_bytes + pairs * 4 + T * H * b, "flops": 2 * pairs * H},
        "layer": {"bytes": touched * 3 * I * H * b + E * H * b + 2 * T * H * b,
                  "flops": 2 * pairs * 3 * H * I + 2 * T * H * E},
        "touched_experts": touched,
    }


def kernel_label(kind: str, block_m: int) -> str:
    """Name of the kernel instance the library launches for a GEMM at a
    row-block size (as rocprofv3 lists it, template arguments shortened)."""
    if kind == "gate_up":
        return {16: "grouped_gemm_skinny_kernel<true,1,2,8,false>", 32: "grouped_gemm_kernel<GemmCfg<32,128,true>,false>",
                64: "grouped_gemm_wide_kernel<WideCfg<true,64,4,2,1,128,2>,false,false,1>",
                128: "grouped_gemm_wide_kernel<WideCfg<true,128,4,4,2,128,1>,false,false,1>",
                256: "grouped_gemm_wide_kernel<WideCfg<true,128,4,4,2,128,1>,false,false,2>"}[block_m]
    return {16: "grouped_gemm_skinny_kernel<false,4,4,4,true>", 32: "grouped_gemm_kernel<GemmCfg<32,128,false>,true>",
            64: "grouped_gemm_wide_kernel<WideCfg<false,64,4,2,1,128,2>,true,false,1>",
            128: "grouped_gemm_wide_kernel<WideCfg<false,128,4,4,2,128,1>,true,true,1>",
            256: "grouped_gemm_wide_kernel<WideCfg<false,128,4,4,2,128,1>,true,true,2>"}[block_m]


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, seconds: float):
    """Oracle tokens/s on the host cores over a bounded sample of the same
    workload (the whole batch repeated, or a prefix of it, for about
    `seconds` of CPU work), and on one core for a quarter of that."""
    import numpy as np

    import oracle

    s = inp.shape
    orc = oracle.default()
    threads = orc.max_threads()

    def rate(budget, nthreads):
        orc.set_threads(nthreads)
        n = min(s.T, 2 * nthreads)  # enough tokens to occupy every thread once the estimate is scaled up
        t0 = time.perf_counter()
        orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob, inp.router_bias, np.arange(n))
        per_token = (time.perf_counter() - t0) / n
        budget_tokens = max(1, int(budget / max(per_token, 1e-9)))
        if budget_tokens >= s.T:
            reps = max(1, budget_tokens // s.T)
            tokens = np.arange(s.T)
            sample = f"whole batch of {s.T} tokens x {reps} repeats"
        else:
            reps = 1
            tokens = np.arange(budget_tokens)
            sample = f"first {budget_tokens} of {s.T} tokens"
        t0 = time.perf_counter()
        for _ in range(reps):
            orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob, inp.router_bias, tokens)
        dt = time.perf_counter() - t0
        return len(tokens) * reps / dt, sample, dt

    try:
        v1, sample1, dt1 = rate(seconds / 4, 1)
        v, sample, dt = rate(seconds, threads)
    finally:
        orc.set_threads(threads)
    return {
        "value": round(v, 3),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{sample}; float64 per-token loop, {dt:.1f} s",
        "cpu_model": host_cpu_model(),
        "one_core": {"value": round(v1, 3), "unit": "tokens/s", "sample": f"{sample1}, {dt1:.1f} s"},
    }


def percentiles(values):
    import numpy as np

    v = np.asarray(values, dtype=np.float64)
    return {"median": round(float(np.median(v)), 5), "p10": round(float(np.percentile(v, 10)), 5),
            "p90": round(float(np.percentile(v, 90)), 5)}


class WeightCache:
    """Expert weights shared by workloads of the same (E, H, I) and seed."""

    def __init__(self):
        self.key, self.value = None, None

    def get(self, shape, seed):
        import synth

        key = (shape.E, shape.H, shape.I, seed)
        if key != self.key:
            self.value = None
            self.value = synth.expert_weights(shape, seed)
            self.key = key
        return self.value


def measure_layer(workload: str, steps: int, warmup: int, seed: int, weights: WeightCache, block_m: int = 0,
                  copies: int = 0):
    """One workload: returns (record, host inputs, block_m)."""
    import numpy as np
    import torch

    import synth
    import sparse_mixture_experts_softmax_amd as moe

    shape = synth.CONFIGS[workload]
    progress(f"{workload}: generating inputs (T={shape.T} H={shape.H} E={shape.E} k={shape.k} I={shape.I})")
    inp = synth.make_inputs(shape, seed=seed, weights=False)
    inp.w13, inp.w2 = weights.get(shape, seed)
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I
    weight_bytes = inp.w13.nbytes + inp.w2.nbytes
    copies = copies or max(1, min(4, -(-(512 << 20) // weight_bytes) + 1))

    def dev(bits):
        return torch.from_numpy(bits).view(torch.bfloat16).to("cuda")

    x = dev(inp.x)
    wr = dev(inp.w_router)
    bias = None if inp.router_bias is None else torch.from_numpy(inp.router_bias).cuda()
    # expert weights are packed once, at load time (outside the timed region)
    packed = moe.pack_experts(dev(inp.w13), dev(inp.w2))
    w13s, w2s = [packed.w13], [packed.w2]
    for _ in range(copies - 1):
        w13s.append(w13s[0].clone())
        w2s.append(w2s[0].clone())
    block_m = block_m or moe.moe_pick_block_m(T, k, E)
    b = moe.allocate(T, H, E, k, I, "cuda", block_m)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    dense = workload == "dense"
    g = b  # the down projection's grouping
    down_bm = block_m
    if dense:
        ids0 = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
        ones = torch.ones((T, 1), dtype=torch.float32, device="cuda")
        # as gated_mlp: with one expert the down projection may take finer row
        # blocks (the grouping is the identity at every block size)
        down_bm = moe.dense_down_block_m(T, H, block_m, torch.cuda.get_device_properties(0).multi_processor_count)
        if down_bm != block_m:
            g = moe.allocate(T, H, E, k, I, "cuda", down_bm)

    def align(w13, w2):
        moe.moe_align_by_expert(ids0 if dense else b.topk_ids, T, k, E, block_m, b.sorted_ids, b.block_expert,
                                b.expert_counts, b.num_padded, b.workspace, sp)
        if g is not b:
            moe.moe_align_by_expert(ids0, T, k, E, down_bm, g.sorted_ids, g.block_expert, g.expert_counts,
                                    g.num_padded, g.workspace, sp)

    calls = [
        lambda w13, w2: None if dense else moe.moe_route(x, wr, bias, b.logits, b.topk_ids, b.topk_weights, T, H, E,
                                                         k, shape.norm_topk_prob, sp),
        align,
        lambda w13, w2: moe.moe_grouped_gemm_gate_up_silu(x, w13, b.sorted_ids, b.block_expert, b.num_padded, T, k,
                                                          H, I, E, block_m, b.cap, b.act, sp),
        lambda w13, w2: moe.moe_grouped_gemm_down(b.act, w2, g.sorted_ids, g.block_expert, g.num_padded, T, k, H, I,
                                                  E, down_bm, g.cap, b.y, sp),
        lambda w13, w2: moe.moe_combine(b.y, ones if dense else b.topk_weights, T, k, H, b.out, sp),
    ]
    gu, dn = KERNELS.index("gate_up"), KERNELS.index("down")

    def new_events():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def step(c, marks=None, step_ev=None):
        """marks: None, or {call index: (event before, event after)}."""
        w13, w2 = w13s[c % copies], w2s[c % copies]
        if step_ev:
            step_ev[0].record(stream)
        for j, call in enumerate(calls):
            if marks and j in marks:
                marks[j][0].record(stream)
            call(w13, w2)
            if marks and j in marks:
                marks[j][1].record(stream)
        if step_ev:
            step_ev[1].record(stream)

    progress(f"{workload}: warmup {warmup} steps (block_m={block_m}, {copies} weight copies)")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    progress(f"{workload}: timing {steps} steps")
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    progress(f"{workload}: timing {steps} steps with events around each step and both GEMMs")
    marks = [{gu: new_events(), dn: new_events()} for _ in range(steps)]
    step_evs = [new_events() for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i, marks[i], step_evs[i])
    torch.cuda.synchronize()
    elapsed_marked = time.perf_counter() - t1
    step_ms = [a.elapsed_time(c) for a, c in step_evs]
    gu_ms = float(np.mean([m[gu][0].elapsed_time(m[gu][1]) for m in marks]))
    dn_ms = float(np.mean([m[dn][0].elapsed_time(m[dn][1]) for m in marks]))

    # A/B: the down projection and the combine as one launch
    # (moe_grouped_gemm_down_combine), same buffers, same number of steps
    fused_ms = None
    if not dense:
        fused_call = lambda w13, w2: moe.moe_grouped_gemm_down_combine(  # noqa: E731
            b.act, w2, b.sorted_ids, b.block_expert, b.num_padded, b.topk_weights, T, k, H, I, E, block_m, b.cap, b.y,
            b.counters, b.out, sp)

        def fused_step(c):
            w13, w2 = w13s[c % copies], w2s[c % copies]
            for call in calls[:3]:
                call(w13, w2)
            fused_call(w13, w2)

        for i in range(warmup):
            fused_step(i)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(steps):
            fused_step(i)
        torch.cuda.synchronize()
        fused_ms = (time.perf_counter() - t2) * 1e3 / steps

    n_break = min(steps, 50)
    all_marks = [{j: new_events() for j in range(len(calls))} for _ in range(n_break)]
    for i in range(n_break):
        step(i, all_marks[i])
    torch.cuda.synchronize()
    per_kernel_ms = {name: float(np.mean([m[j][0].elapsed_time(m[j][1]) for m in all_marks]))
                     for j, name in enumerate(KERNELS)}
    ms_per_step = elapsed * 1e3 / steps
    counts = b.expert_counts.cpu().numpy()
    work = algorithmic_work(shape, counts, b.y.element_size())
    if dense:
        work["layer"]["flops"] -= 2 * T * H * E  # no router

    bound = "hbm" if workload in ("decode", "tiny", "medium") else "mfma"

    def roofline(kind, kern_ms):
        s = kern_ms * 1e-3
        if bound == "hbm":
            achieved = work[kind]["bytes"] / s / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                 "frac": round(achieved / PEAK_HBM_GBPS, 4)}
        else:
            achieved = work[kind]["flops"] / s / 1e12
            r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        rec = counter_record(workload, kind)
        r["kernel"] = f"moe_grouped_gemm_{'gate_up_silu' if kind == 'gate_up' else 'down'}: " + \
            kernel_label(kind, down_bm if kind == "down" else block_m)
        r["kernel_ms"] = round(kern_ms, 5)
        r["timing"] = (f"HIP events around each of the {steps} launches in a second timed region of {steps} steps "
                       f"({elapsed_marked * 1e3 / steps:.4f} ms/step with the markers)")
        r["algorithmic_per_launch"] = work[kind]["bytes"] if bound == "hbm" else work[kind]["flops"]
        r["algorithmic_bytes_per_launch"] = work[kind]["bytes"]
        r["traffic"] = rec.get("hbm_bytes_per_launch") if rec else None
        r["mfma_busy"] = rec.get("mfma_busy_frac") if rec else None
        r["counters"] = rec.get("summary") if rec else None
        return r

    layer_s = ms_per_step * 1e-3
    record = {
        "workload": WORKLOAD_TEXT[workload],
        "name": workload,
        "T": T, "hidden": H, "experts": E, "top_k": k, "intermediate": I, "norm_topk_prob": shape.norm_topk_prob,
        "block_m": block_m, "down_block_m": down_bm, "weight_copies_rotated": copies,
        "touched_experts": work["touched_experts"],
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(T / layer_s, 1),
        "step_ms_events": percentiles(step_ms),
        "layer": {
            "hbm_GBps": round(work["layer"]["bytes"] / layer_s / 1e9, 1),
            "hbm_frac": round(work["layer"]["bytes"] / layer_s / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_TFLOPs": round(work["layer"]["flops"] / layer_s / 1e12, 2),
            "mfma_frac": round(work["layer"]["flops"] / layer_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_ms_events": {n: round(v, 5) for n, v in per_kernel_ms.items()},
        },
        "roofline": roofline("gate_up", gu_ms),
        "down_roofline": roofline("down", dn_ms),
        "fused_combine": None if fused_ms is None else {
            "ms_per_step": round(fused_ms, 5), "tokens_per_s": round(T / (fused_ms * 1e-3), 1),
            "note": "down projection and weighted combine as one launch (moe_grouped_gemm_down_combine), "
                    f"{steps} steps timed like ms_per_step"},
    }
    del packed, w13s, w2s, b, g, x, wr
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return record, inp


def norm_bench(args):
    """The fused residual add + RMSNorm that precedes the layer, in place on a
    [4096, 2048] bf16 hidden state: HBM-bound (reads x and the residual,
    writes both)."""
    import numpy as np
    import torch

    import synth
    import sparse_mixture_experts_softmax_amd as moe

    T, H = NORM_SHAPE
    progress(f"add_rmsnorm T={T} H={H}")
    xb = synth.normal_bf16(args.seed, synth.TAG_X, (T, H), 1.0)
    rb = synth.normal_bf16(args.seed, 0x200, (T, H), 1.0)
    wb = synth.normal_bf16(args.seed, 0x201, (H,), 1.0)
    dev = lambda a: torch.from_numpy(a).view(torch.bfloat16).cuda()  # noqa: E731
    x, r, w = dev(xb), dev(rb), dev(wb)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        moe.moe_fused_add_rmsnorm(x, r, w, T, H, 1e-6, True, sp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    kern = [a.elapsed_time(b) for a, b in evs]
    kern_ms = float(np.mean(kern))
    nbytes = 4 * T * H * 2 + H * 2
    ms = elapsed * 1e3 / args.steps
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": "fused residual add + RMSNorm tokens/s; achieved HBM GB/s",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) hidden state and residual)",
        "config": {"workload": WORKLOAD_TEXT["add_rmsnorm"], "T": T, "hidden": H, "eps": 1e-6},
        "step_ms_events": percentiles(kern),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": "fused_add_rmsnorm_kernel<1>",
                     "kernel_ms": round(kern_ms, 5), "algorithmic_per_launch": nbytes, "traffic": None},
    }
    result["norm_route_ab"] = norm_route_ab(args)
    if args.cpu_seconds > 0:
        import oracle

        n = 256
        t1 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t1 < min(args.cpu_seconds, 5.0):
            oracle.fused_add_rmsnorm(xb[:n], rb[:n], wb, 1e-6)
            reps += 1
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(n * reps / dt, 1), "unit": "tokens/s",
                                  "cores": oracle.default().max_threads(), "kind": "oracle",
                                  "sample": f"first {n} rows x {reps} repeats, {dt:.1f} s",
                                  "cpu_model": host_cpu_model()}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def norm_route_ab(args):
    """The residual add + RMSNorm before the router, as the standalone kernel
    followed by moe_route, against moe_fused_add_rmsnorm_route (the norm
    inside the router's read of x), at the decode and prefill shapes
    (E = 128, k = 8): mean microseconds per pair of calls / per fused call,
    HIP events around each of K repetitions."""
    import numpy as np
    import torch

    import synth
    import sparse_mixture_experts_softmax_amd as moe

    out = {}
    for name, T in (("decode", 64), ("prefill", 4096)):
        H, E, k = 2048, 128, 8
        dev = lambda a: torch.from_numpy(a).view(torch.bfloat16).cuda()  # noqa: E731
        x = dev(synth.normal_bf16(args.seed, synth.TAG_X, (T, H), 1.0))
        r = dev(synth.normal_bf16(args.seed, 0x200, (T, H), 1.0))
        w = dev(synth.normal_bf16(args.seed, 0x201, (H,), 1.0))
        wr = dev(synth.normal_bf16(args.seed, synth.TAG_WR, (E, H), 0.02))
        xs, rs = x.clone(), r.clone()
        xo, ro = torch.empty_like(x), torch.empty_like(x)
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        sp = stream.cuda_stream

        def separate():
            moe.moe_fused_add_rmsnorm(xs, rs, w, T, H, 1e-6, True, sp)
            moe.moe_route(xs, wr, None, lg, ids, wt, T, H, E, k, True, sp)

        def fused():
            moe.moe_fused_add_rmsnorm_route(x, r, w, 1e-6, True, xo, ro, wr, None, lg, ids, wt, T, H, E, k, True, sp)

        res = {}
        for label, fn in (("separate_us", separate), ("fused_us", fused)):
            for _ in range(args.warmup + 10):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for a, b in evs:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            res[label] = round(float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3, 2)
        res["T"] = T
        out[name] = res
        progress(f"norm + route {name}: separate {res['separate_us']} us, fused {res['fused_us']} us")
    return out


def copy_calibration(mb: int):
    """A plain device-to-device copy of `mb` MiB, for scaling HBM counters."""
    import torch

    n = mb * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


# ----------------------------------------------------------------------------
# Counter records (rocprofv3 --pmc passes -> profiles/counters.json)
# ----------------------------------------------------------------------------
COPY_MB = 1024
PASSES = {
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
    "mfma": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
}


def counter_commands(workload: str):
    """The rocprofv3 counter passes behind a workload's record: one run per
    pass (counters within one block's limits), output under DIR."""
    run = f"python3 -u bench.py --workload {workload} --also none --steps 10 --warmup 2 --cpu-seconds 0"
    cmds = [f"rocprofv3 --pmc {ctr} --output-format csv -d DIR -o {workload}_{p} -- {run}"
            for p, ctr in PASSES.items()]
    for p in ("fetch", "write"):
        cmds.append(f"rocprofv3 --pmc {PASSES[p]} --output-format csv -d DIR -o copy_{p} -- "
                    f"python3 -u bench.py --copy-calibration-mb {COPY_MB}")
    return cmds


def _pmc(directory: str, prefix: str):
    """{kernel name: {counter: mean value per dispatch}} from one pass."""
    files = glob.glob(os.path.join(directory, "**", f"{prefix}_counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {prefix}_counter_collection.csv under {directory}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].split("(")[0]
                key = (name, r.get("Dispatch_Id") or r.get("Correlation_Id", ""), r["Counter_Name"])
                acc.setdefault(key, 0.0)
                acc[key] += float(r["Counter_Value"])
    per = {}
    for (name, _disp, ctr), v in acc.items():
        per.setdefault(name, {}).setdefault(ctr, []).append(v)
    return {name: {c: sum(v) / len(v) for c, v in d.items()} for name, d in per.items()}


def _stats(directory: str, prefix: str):
    files = glob.glob(os.path.join(directory, "**", f"{prefix}_kernel_stats.csv"), recursive=True)
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out[r["Name"].split("(")[0]] = float(r["AverageNs"]) / 1e3
    return out


def stats_command(workload: str) -> str:
    return (f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o {workload} -- python3 -u bench.py "
            f"--workload {workload} --also none --steps 50 --warmup 20 --cpu-seconds 0")


def record_stats(directory: str, workload: str):
    """profiles/<workload>_kernel_stats.md from the kernel-trace run of
    ``stats_command(workload)``."""
    import synth

    files = glob.glob(os.path.join(directory, "**", f"{workload}_kernel_stats.csv"), recursive=True)
    if not files:
        return
    shape = synth.CONFIGS[workload]
    lines = [f"# rocprofv3 kernel statistics: {WORKLOAD_TEXT[workload]} (T={shape.T}, H={shape.H}, E={shape.E}, "
             f"k={shape.k}, I={shape.I})", "",
             "Whole bench run (20 warm-up and 3 x 50 timed steps of the layer, 20 + 50 steps with the down "
             "projection and the combine fused, plus the one-time weight packing and copies), "
             "from the repository root on one MI355X (`export TMPDIR=/tmp` first; DIR = the output directory):", "",
             "```", stats_command(workload), "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def record_counters(directory: str, workload: str):
    """Parse the counter passes of ``counter_commands(workload)`` from
    ``directory`` into profiles/counters.json and a summary table."""
    import numpy as np

    import synth
    import sparse_mixture_experts_softmax_amd as moe

    cf, cw = _pmc(directory, "copy_fetch"), _pmc(directory, "copy_write")
    copy_name = next(n for n in cf if "copyBuffer" in n or "copy" in n.lower())
    nbytes = COPY_MB * 1024 * 1024
    f_fac = nbytes / (cf[copy_name]["FETCH_SIZE"] * 1024)
    w_fac = nbytes / (cw[copy_name]["WRITE_SIZE"] * 1024)
    fe, wr, mf = (_pmc(directory, f"{workload}_{p}") for p in ("fetch", "write", "mfma"))
    shape = synth.CONFIGS[workload]
    bm = moe.moe_pick_block_m(shape.T, shape.k, shape.E)
    try:
        with open(COUNTERS_FILE) as fh:
            db = json.load(fh)
    except (OSError, ValueError):
        db = {}
    summary = f"profiles/{workload}_counters.md"
    lines = [f"# rocprofv3 counters per launch: {WORKLOAD_TEXT[workload]} "
             f"(T={shape.T}, H={shape.H}, E={shape.E}, k={shape.k}, I={shape.I}, block_m {bm})", "",
             "One run per counter pass, from the repository root on one MI355X "
             "(`cd /tmp && export TMPDIR=/tmp` first; DIR = the output directory):", "", "```",
             *counter_commands(workload), "```", "",
             f"HBM bytes: a plain device copy of {COPY_MB} MiB (`{copy_name}`) reads FETCH_SIZE = "
             f"{cf[copy_name]['FETCH_SIZE']:.0f} KiB and WRITE_SIZE = {cw[copy_name]['WRITE_SIZE']:.0f} KiB per "
             f"launch, so fetched bytes = FETCH_SIZE x 1024 x {f_fac:.3f} and written bytes = WRITE_SIZE x 1024 x "
             f"{w_fac:.3f}. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), "
             "GRBM_GUI_ACTIVE summing the 8 XCDs' busy cycles.", "",
             "| kernel | step | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) | MFMA busy |",
             "|---|---|---|---|---|---|"]
    for kind in ("gate_up", "down", "down_combine", "combine", "route", "align"):
        names = [n for n in fe if _kind_of(n) == kind]
        for n in names:
            fb = fe[n]["FETCH_SIZE"] * 1024 * f_fac
            wb = wr.get(n, {}).get("WRITE_SIZE", float("nan")) * 1024 * w_fac
            m = mf.get(n, {})
            busy = None
            if m.get("GRBM_GUI_ACTIVE"):
                busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * m["GRBM_GUI_ACTIVE"] / 8)
            lines.append(f"| `{n}` | {kind} | {fe[n]['FETCH_SIZE']:.0f} | {wr.get(n, {}).get('WRITE_SIZE', 0):.0f} | "
                         f"{fb + wb:.4g} ({fb:.4g} read + {wb:.4g} written) | "
                         f"{'' if busy is None else f'{busy:.1%}'} |")
            if kind in KERNEL_SOURCES and len(names) == 1:
                db[f"{workload}/{kind}"] = {
                    "source_sha": source_hash(kind), "kernel": n, "hbm_bytes_per_launch": int(round(fb + wb)),
                    "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
                    "mfma_busy_frac": None if busy is None else round(busy, 4), "summary": summary,
                }
    with open(os.path.join(ROOT, summary), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(dict(sorted(db.items())), fh, indent=1)
        fh.write("\n")
    print("\n".join(lines))
    del np


def _kind_of(kernel_name: str) -> str:
    """Which step a kernel of the library belongs to, from its name (the
    GEMMs' first boolean template argument is true for gate/up; their last
    one is nonzero when the weighted combine is fused into the down
    projection, moe_grouped_gemm_down_combine)."""
    if "grouped_gemm" in kernel_name:
        m = re.search(r"(?:WideCfg<|skinny_kernel<|GemmCfg<\d+, \d+, )(true|false)", kernel_name)
        if m and m.group(1) == "true":
            return "gate_up"
        last = re.search(r",\s*(\d+)>\s*$", kernel_name)
        return "down_combine" if last and last.group(1) != "0" else "down"
    for kind, pat in (("combine", "combine"), ("route", "router"), ("route", "topk"), ("align", "align")):
        if pat in kernel_name:
            return kind
    return "other"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--also", default="medium,prefill,skewed,large",
                    help="further workloads measured in the same run and reported under 'workloads' "
                         "(comma-separated; 'none' for none)")
    ap.add_argument("--also-steps", type=int, default=100, help="timed steps of each of those workloads")
    ap.add_argument("--also-warmup", type=int, default=30,
                    help="untimed steps before them (a fresh process runs its first ~20 steps slower)")
    ap.add_argument("--copies", type=int, default=0, help="resident weight copies rotated over steps (0 = auto)")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget; 0 skips it")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0)
    ap.add_argument("--record-counters", default="", metavar="DIR")
    args = ap.parse_args()

    if args.record_counters:
        record_stats(args.record_counters, args.workload)
        record_counters(args.record_counters, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_softmax_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.lib()  # fail loudly if the HIP library is not built
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)
        return
    if args.workload == "add_rmsnorm":
        norm_bench(args)
        return

    weights = WeightCache()
    head, inp = measure_layer(args.workload, args.steps, args.warmup, args.seed, weights, args.block_m, args.copies)
    also = [w for w in args.also.split(",") if w and w != "none" and w != args.workload]
    extra = {}
    for w in also:
        if w not in WORKLOAD_TEXT or w == "add_rmsnorm":
            raise SystemExit(f"--also: unknown workload {w}")
        rec, _ = measure_layer(w, args.also_steps, args.also_warmup, args.seed, weights)
        extra[w] = rec

    roof = head.pop("roofline")
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, bf16)",
        "config": {key: head[key] for key in ("workload", "T", "hidden", "experts", "top_k", "intermediate",
                                              "norm_topk_prob", "block_m", "weight_copies_rotated",
                                              "touched_experts")},
        "roofline": roof,
        "step_ms_events": head["step_ms_events"],
        "layer": head["layer"],
        "down_roofline": head["down_roofline"],
        "fused_combine": head["fused_combine"],
        "workloads": extra,
    }
    if args.cpu_seconds > 0:
        progress(f"CPU baseline (oracle, ~{args.cpu_seconds:.0f} s on all host threads, then one thread)")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", "")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
