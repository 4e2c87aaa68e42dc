#!/usr/bin/env python3
"""Throughput of the fused sparse MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

A step is one pass of the whole layer (route, align, gate/up GEMM + SiLU*mul,
down GEMM, combine: the five C-ABI calls) over one batch of synthetic
inputs already resident in HBM (expert weights packed once, at load time).
W untimed steps, then exactly K timed steps between two device
synchronisations, with nothing else on the stream; the weights are rotated
over ``--copies`` resident copies so the 256 MB Infinity Cache cannot serve
one step's weights to the next. Event markers between kernels cost several
microseconds each on this stream, so they are kept out of that region: a
second timed region runs the same K steps with HIP events recorded on the
launch stream around the dominant kernel only, giving its average duration
for the roofline entry (its algorithmic bytes or flops per launch over that
duration); a third, short pass with events around every call gives the
per-kernel breakdown. The CPU oracle is timed on a bounded sample of the
same workload on the host cores (cpu_baseline).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
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
    "dense": "dense SwiGLU GatedMLP (Qwen3-0.6B MLP shape) through the grouped GEMMs",
    "add_rmsnorm": "fused residual add + RMSNorm before the layer (prefill-shaped hidden state)",
}
NORM_SHAPE = (4096, 2048)  # tokens, hidden (the prefill-shaped layer's input)
KERNELS = ["route", "align", "gate_up", "down", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
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


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, or None when
    absent or taken on a different version of the kernel's source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(f"{workload}/{kernel}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


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


def cpu_baseline(inp, seconds: float):
    """Oracle tokens/s on the host cores over a bounded sample of the same
    workload: the whole batch repeated, or a prefix of it, for about
    `seconds` of CPU work."""
    import numpy as np

    import oracle

    s = inp.shape
    orc = oracle.default()
    n = min(s.T, 2 * orc.max_threads())  # enough tokens to occupy every thread once the estimate is scaled up
    t0 = time.perf_counter()
    orc.moe_layer(inp.x, inp.w_router, inp.w13, inp.w2, s.k, s.norm_topk_prob, inp.router_bias, np.arange(n))
    per_token = (time.perf_counter() - t0) / n
    budget_tokens = max(1, int(seconds / max(per_token, 1e-9)))
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
    return {
        "value": round(len(tokens) * reps / dt, 3),
        "unit": "tokens/s",
        "cores": orc.max_threads(),
        "kind": "oracle",
        "sample": f"{sample}; float64 per-token loop, {dt:.1f} s",
    }


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
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = 4 * T * H * 2 + H * 2
    ms = elapsed * 1e3 / args.steps
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": "fused residual add + RMSNorm tokens/s; achieved HBM GB/s",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) hidden state and residual)",
        "config": {"workload": WORKLOAD_TEXT["add_rmsnorm"], "T": T, "hidden": H, "eps": 1e-6},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": "fused_add_rmsnorm_kernel<1>",
                     "kernel_ms": round(kern_ms, 5), "algorithmic_per_launch": nbytes, "traffic": None},
    }
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
                                  "sample": f"first {n} rows x {reps} repeats, {dt:.1f} s"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--copies", type=int, default=0, help="resident weight copies rotated over steps (0 = auto)")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget; 0 skips it")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
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

    shape = synth.CONFIGS[args.workload]
    progress(f"generating {args.workload} inputs (T={shape.T} H={shape.H} E={shape.E} k={shape.k} I={shape.I})")
    inp = synth.make_inputs(shape, seed=args.seed)
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.k, shape.I
    weight_bytes = (inp.w13.nbytes + inp.w2.nbytes)
    copies = args.copies or max(1, min(4, -(-(512 << 20) // weight_bytes) + 1))

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
    block_m = args.block_m or moe.moe_pick_block_m(T, k, E)
    b = moe.allocate(T, H, E, k, I, "cuda", block_m)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    dense = args.workload == "dense"
    if dense:
        ids0 = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
        ones = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    calls = [
        lambda w13, w2: None if dense else moe.moe_route(x, wr, bias, b.logits, b.topk_ids, b.topk_weights, T, H, E, k,
                                      shape.norm_topk_prob, sp),
        lambda w13, w2: moe.moe_align_by_expert(ids0 if dense else b.topk_ids, T, k, E, block_m, b.sorted_ids,
                                                b.block_expert, b.expert_counts, b.num_padded, b.workspace, sp),
        lambda w13, w2: moe.moe_grouped_gemm_gate_up_silu(x, w13, b.sorted_ids, b.block_expert, b.num_padded, T, k,
                                                          H, I, E, block_m, b.cap, b.act, sp),
        lambda w13, w2: moe.moe_grouped_gemm_down(b.act, w2, b.sorted_ids, b.block_expert, b.num_padded, T, k, H, I,
                                                  E, block_m, b.cap, b.y, sp),
        lambda w13, w2: moe.moe_combine(b.y, ones if dense else b.topk_weights, T, k, H, b.out, sp),
    ]
    dom_idx = KERNELS.index("gate_up")

    def step(c, marks=None):
        """marks: None, or {call index: (event before, event after)}."""
        w13, w2 = w13s[c % copies], w2s[c % copies]
        for j, call in enumerate(calls):
            if marks and j in marks:
                marks[j][0].record(stream)
            call(w13, w2)
            if marks and j in marks:
                marks[j][1].record(stream)

    def new_events():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    progress(f"warmup {args.warmup} steps (block_m={block_m}, {copies} weight copies)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    progress(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    progress(f"timing {args.steps} steps with events around the dominant kernel")
    dom_marks = [{dom_idx: new_events()} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(i, dom_marks[i])
    torch.cuda.synchronize()
    elapsed_marked = time.perf_counter() - t1
    dom_ms = float(np.mean([m[dom_idx][0].elapsed_time(m[dom_idx][1]) for m in dom_marks]))

    n_break = min(args.steps, 50)
    all_marks = [{j: new_events() for j in range(len(calls))} for _ in range(n_break)]
    for i in range(n_break):
        step(i, all_marks[i])
    torch.cuda.synchronize()
    per_kernel_ms = {name: float(np.mean([m[j][0].elapsed_time(m[j][1]) for m in all_marks]))
                     for j, name in enumerate(KERNELS)}
    ms_per_step = elapsed * 1e3 / args.steps
    counts = b.expert_counts.cpu().numpy()
    work = algorithmic_work(shape, counts, b.y.element_size())

    bound = "hbm" if args.workload in ("decode", "tiny") else "mfma"
    if dense:
        work["layer"]["flops"] -= 2 * T * H * E  # no router
    dom = "gate_up"
    dom_s = dom_ms * 1e-3
    if bound == "hbm":
        achieved = work[dom]["bytes"] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    else:
        achieved = work[dom]["flops"] / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["kernel"] = ("moe_grouped_gemm_gate_up_silu: " +
                      {16: "grouped_gemm_skinny_kernel<true,1,2,8>", 32: "grouped_gemm_kernel<GemmCfg<32,128,true>>",
                       64: "grouped_gemm_wide_kernel<WideCfg<true,64,4,4,2,128>,false,false>",
                       128: "grouped_gemm_wide_kernel<WideCfg<true,128,4,4,2,128>,false,false>"}[block_m])
    roof["kernel_ms"] = round(dom_ms, 5)
    roof["timing"] = (f"HIP events around each of the {args.steps} launches in a second timed region of "
                      f"{args.steps} steps ({elapsed_marked * 1e3 / args.steps:.4f} ms/step with the markers)")
    roof["algorithmic_per_launch"] = work[dom]["bytes"] if bound == "hbm" else work[dom]["flops"]
    roof["traffic"] = measured_traffic(args.workload, dom)

    layer_s = ms_per_step * 1e-3
    result = {
        "metric": METRIC,
        "value": round(T / layer_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, bf16)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": T, "hidden": H, "experts": E, "top_k": k,
                   "intermediate": I, "norm_topk_prob": shape.norm_topk_prob, "block_m": block_m,
                   "weight_copies_rotated": copies, "touched_experts": work["touched_experts"]},
        "roofline": roof,
        "layer": {
            "hbm_GBps": round(work["layer"]["bytes"] / layer_s / 1e9, 1),
            "hbm_frac": round(work["layer"]["bytes"] / layer_s / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_TFLOPs": round(work["layer"]["flops"] / layer_s / 1e12, 2),
            "mfma_frac": round(work["layer"]["flops"] / layer_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_ms_events": {n: round(v, 5) for n, v in per_kernel_ms.items()},
        },
    }
    if args.cpu_seconds > 0:
        progress(f"CPU baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", "")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
