"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]

One step is one pass of the whole path over one batch of synthetic input:
route + indices->multihot + align + multihot->indices (one call,
moe_route_align_inverse: one kernel for at most 512 routing slots, else a
route kernel that also counts the alignment's histograms plus the scatter
kernel, whose launch also carries the inverse conversion's blocks) ->
grouped FC1 + SiLU-and-mul -> grouped FC2 -> combine (decode workloads use
the decode FFN kernels: FC2 and the combine through moe_ffn_down_combine and,
for the smallest batches, the routing calls and FC1 as one call,
moe_route_align_gate_up, one launch each).  Inputs are resident in HBM before timing starts; nothing is
allocated inside the timed region.  Each phase is bracketed by HIP events on
the stream the library launches on (torch's current stream), so per-kernel
durations are measured live.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + % bf16 MFMA peak (prefill), % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = {
    "gate_up": "mixture_experts_routing_moe_amd/csrc/gemm_bf16.hip",
    "decode_gate_up": "mixture_experts_routing_moe_amd/csrc/decode.hip",
    # route + align + the maps and their inverse + decode FC1 in one launch
    "decode_route_gate_up": ["mixture_experts_routing_moe_amd/csrc/decode.hip",
                             "mixture_experts_routing_moe_amd/csrc/moe_internal.h"],
    # decode FC2 + combine (one launch for the smallest batches, else two)
    "decode_down_combine": ["mixture_experts_routing_moe_amd/csrc/decode.hip",
                            "mixture_experts_routing_moe_amd/csrc/combine.hip"],
    # route_hist_kernel + align_scatter_kernel with the inverse's blocks (the
    # routing rows of moe_route_align_inverse)
    "route_align_inverse": ["mixture_experts_routing_moe_amd/csrc/align.hip",
                            "mixture_experts_routing_moe_amd/csrc/moe_internal.h"],
    "ffn_backward": ["mixture_experts_routing_moe_amd/csrc/backward.hip",
                     "mixture_experts_routing_moe_amd/csrc/gemm_bf16.hip"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral",
                   choices=["mixtral", "finegrained", "decode1", "decode32", "routing",
                            "grouped_noaux", "grouped_greedy", "router_finegrained",
                            "router_mixtral", "backward_mixtral", "backward_finegrained"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", type=int, default=None,
                   help="1: time the whole step as one captured HIP graph replay (the "
                        "per-phase breakdown still comes from eager launches); default 1 "
                        "for the decode and routing-only workloads, whose steps are "
                        "launch-bound, else 0")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy 5 times and exit: the "
                        "known-size kernel that calibrates the HBM byte counters")
    p.add_argument("--draws", type=int, default=None,
                   help="distinct routing draws rotated over the steps (default: 32 for "
                        "decode workloads, else 1)")
    p.add_argument("--flush", type=int, default=None,
                   help="1: overwrite a 512 MiB buffer before every step (outside the "
                        "per-kernel events) so weights come from HBM, not the Infinity "
                        "Cache; ms_per_step is then the sum of the kernel phases "
                        "(default: 1 for the decode and routing-only workloads, else 0)")
    return p.parse_args()


def source_hash(rel) -> str:
    """First 16 hex digits of the SHA-256 of one source file, or of several in order."""
    h = hashlib.sha256()
    for r in [rel] if isinstance(rel, str) else rel:
        with open(os.path.join(ROOT, r), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if kernel not in KERNEL_SRC or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SRC[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s=(10.0, 30.0)):
    """The oracle on a growing prefix of the workload's tokens until ~10 s of
    CPU work (or the whole workload): route + align, then the expert FFN and
    combine for layer workloads, or the multihot conversion and its inverse
    for the routing-only one, all in float64."""
    import numpy as np

    import oracle

    threads = len(os.sched_getaffinity(0))
    has_ffn = "hidden" in inp
    grouped = hasattr(w, "n_group")

    router = "w_gate" in inp

    def run(n):
        t0 = time.perf_counter()
        if router:
            lg = oracle.router_logits(inp["hidden"][:n], inp["w_gate"], "bf16")
            oracle.route(lg.astype(np.float32), w.k, w.norm)
            return time.perf_counter() - t0
        if grouped:
            tw, ids = oracle.route_grouped(inp["logits"][:n], w.k, w.n_group, w.topk_group,
                                           w.method, bias=inp["bias"], renormalize=w.renorm)
        else:
            tw, ids = oracle.route(inp["logits"][:n], w.k, w.norm)
        oracle.align(ids, w.E)
        if has_ffn:
            oracle.expert_ffn(inp["hidden"][:n], inp["w13"], inp["w2"], tw, ids,
                              "bf16" if w.dtype == "bf16" else "f32", threads=threads)
        else:
            _, pim, pos = oracle.indices_to_multihot(ids, tw, w.E)
            oracle.multihot_to_indices(pim, pos, w.k)
        return time.perf_counter() - t0

    n, spent = 1, 0.0
    while True:
        n = min(n, w.T)
        dt = run(n)
        spent += dt
        if dt >= budget_s[0] or n >= w.T or spent >= budget_s[1]:
            break
        grow = max(2, int(budget_s[0] / max(dt, 1e-3)))
        n = n * min(grow, 8)
    # A whole workload that takes well under the budget is repeated.
    passes, t_total = 1, dt
    while t_total < budget_s[0] and spent < budget_s[1]:
        dt = run(n)
        spent += dt
        passes += 1
        t_total += dt
    what = ("route + align + expert FFN + combine" if has_ffn and not router else
            "router logits + route" if router else
            f"{'grouped ' if grouped else ''}route + align + indices->multihot + "
            "multihot->indices")
    return {"value": n * passes / t_total, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens x {passes} pass(es): {what} in float64, "
                      f"{t_total:.1f} s on {cpu_model()}"}


def bench_router(args, w, dev):
    """Router GEMM + gating top-k (moe_router_route) on a layer workload's
    hidden states and a seeded linear gate; HBM roofline over its bytes."""
    import numpy as np
    import torch

    import mixture_experts_routing_moe_amd as moe
    import moe_inputs as mi

    T, H, E, k = w.T, w.H, w.E, w.k
    hid = mi.normal_bf16(w.wid, mi.S_HIDDEN, T * H, 1.0).reshape(T, H)
    wg = mi.router_weights(w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, wgd = bf(hid), bf(wg)
    out = (torch.empty((T, E), dtype=torch.float32, device=dev),
           torch.empty((T, k), dtype=torch.float32, device=dev),
           torch.empty((T, k), dtype=torch.int32, device=dev))
    flush_buf = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        moe.moe_router_route(x, wgd, k, w.norm, out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for st in range(args.steps):
        flush_buf.fill_(float(st))  # weights and tokens come from HBM
        ev[st][0].record()
        moe.moe_router_route(x, wgd, k, w.norm, out)
        ev[st][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    nbytes = T * H * 2 + E * H * 2 + T * E * 4 + T * k * 8
    achieved = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC, "value": round(T * 1e3 / ms, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generators, random-init weights)",
        "config": {"workload": f"router_{w.name}", "T": T, "H": H, "E": E, "top_k": k,
                   "norm_topk_prob": w.norm, "cache_flush_between_steps": True,
                   "step_timing": "eager", "path_bytes": nbytes},
        "roofline": {"kernel": "router_route_kernel", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "phase_ms": {"router_route": round(ms, 4)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, {"hidden": hid, "w_gate": wg})
    print(json.dumps(rec), flush=True)


def bench_backward(args, w, dev):
    """Layer backward on a layer workload: moe_expert_ffn_backward (gradients of
    hidden, w13, w2 and the routing weights) then moe_route_backward (the
    logits' gradient), from the saved forward routing and a seeded grad_out.
    MFMA roofline over the five grouped products of the FFN backward."""
    import numpy as np
    import torch

    import mixture_experts_routing_moe_amd as moe
    import moe_inputs as mi

    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    inp = mi.layer_inputs(w)
    gout = mi.grad_output(w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w13, w2, dy = bf(inp["hidden"]), bf(inp["w13"]), bf(inp["w2"]), bf(gout)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    # The forward's routing and alignment, saved (outside the timed steps).
    topk_w, topk_ids = moe.moe_route(logits, k, w.norm)
    aligned = moe.moe_align(topk_ids, E)
    f32 = dict(dtype=torch.float32, device=dev)
    grads = {"grad_hidden": torch.empty((T, H), **f32),
             "grad_w13": torch.empty((E, 2 * I, H), **f32),
             "grad_w2": torch.empty((E, H, I), **f32),
             "grad_topk_w": torch.empty((T, k), **f32)}
    grad_logits = torch.empty((T, E), **f32)
    ws = torch.empty(moe.moe_expert_ffn_backward_workspace_size(T, H, I, E, k),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        moe.moe_expert_ffn_backward(x, w13, w2, topk_w, aligned, dy, grads, ws)
        if ev:
            ev[1].record()
        moe.moe_route_backward(logits, topk_ids, topk_w, grads["grad_topk_w"], w.norm,
                               grad_logits)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(ev[st])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ffn_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    route_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    ms = sum(e[0].elapsed_time(e[2]) for e in ev) / args.steps
    P = T * k
    flops = 16.0 * P * H * I  # gate/up recompute 4PHI, G 2PHI, dx 4PHI, dw2 2PHI, dw13 4PHI
    achieved = flops / (ffn_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(T * 1e3 / ms, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generators, random-init weights)",
        "config": {"workload": f"backward_{w.name}", "T": T, "H": H, "I": I, "E": E,
                   "top_k": k, "norm_topk_prob": w.norm, "step_timing": "eager",
                   "wall_ms_per_step": round(wall_ms, 4),
                   "backward_tflop_per_step": round(flops / 1e12, 3)},
        "roofline": {"kernel": "moe_expert_ffn_backward (5 grouped bf16 GEMMs + 2 row kernels)",
                     "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("ffn_backward", w.name)},
        "phase_ms": {"ffn_backward": round(ffn_ms, 4), "route_backward": round(route_ms, 4)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_backward(w, inp, gout)
    print(json.dumps(rec), flush=True)


def cpu_baseline_backward(w, inp, gout, budget_s=(10.0, 30.0)):
    """The oracle's layer backward (route, FFN backward with weight gradients,
    gating backward; float64) on a growing prefix of the tokens.  With weight
    gradients the oracle visits tokens one after another on one thread."""
    import numpy as np

    import oracle

    def run(n):
        t0 = time.perf_counter()
        tw, ids = oracle.route(inp["logits"][:n], w.k, w.norm)
        g = oracle.expert_ffn_backward(inp["hidden"][:n], inp["w13"], inp["w2"], tw, ids,
                                       gout[:n], "bf16", weights=True)
        oracle.route_backward(inp["logits"][:n], ids, g["grad_topk_w"], w.norm)
        return time.perf_counter() - t0

    n, spent = 1, 0.0
    while True:
        dt = run(n)
        spent += dt
        if dt >= budget_s[0] or n >= w.T or spent >= budget_s[1]:
            break
        n = min(w.T, n * min(8, max(2, int(budget_s[0] / max(dt, 1e-3)))))
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens: route + expert FFN backward with weight "
                      f"gradients + gating backward in float64, {dt:.1f} s on {cpu_model()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 4,
                          "copy_probe_bytes_written": dst.numel() * 4}), flush=True)
        return

    import mixture_experts_routing_moe_amd as moe
    import moe_inputs as mi

    grouped = args.workload in mi.GROUPED
    router = args.workload.startswith("router_")
    backward = args.workload.startswith("backward_")
    if grouped:
        w = mi.GROUPED[args.workload]
    elif router or backward:
        w = mi.WORKLOADS[args.workload.split("_", 1)[1]]
    else:
        w = mi.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if router:
        return bench_router(args, w, dev)
    if backward:
        return bench_backward(args, w, dev)
    if grouped:
        # Group-limited routing: [T, E] scores and (noaux_tc) the correction bias.
        inp = {"logits": mi.grouped_scores(w), "bias": mi.correction_bias(w)}
        bias_d = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev)
    else:
        inp = mi.layer_inputs(w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    T, E, k = w.T, w.E, w.k
    decode = w.name.startswith("decode")
    draws = args.draws if args.draws is not None else (32 if decode else 1)
    routing_only = grouped or w.H == 0
    flush = bool(args.flush if args.flush is not None else (decode or routing_only))
    use_graph = bool(args.graph if args.graph is not None else (decode or routing_only))
    def draw(r):
        if r == 0:
            return inp["logits"]
        return mi.grouped_scores(w, draw=r) if grouped else mi.gating_logits_draw(w, r)

    logits_draws = [torch.from_numpy(draw(r)).to(dev) for r in range(draws)]
    flush_buf = torch.empty(128 << 20, dtype=torch.float32, device=dev) if flush else None
    has_ffn = "hidden" in inp

    # --- every buffer allocated up front -------------------------------------
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    aligned = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_token_ids": torch.empty(T * k, dtype=torch.int32, device=dev),
        "sorted_slot_ids": torch.empty(T * k, dtype=torch.int32, device=dev),
        "slot_to_sorted": torch.empty(T * k, dtype=torch.int32, device=dev),
    }
    align_ws = torch.empty(max(1, moe.moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                           device=dev)
    mh = torch.empty((T, E), dtype=torch.uint8, device=dev)
    pim = torch.empty((T, E), dtype=torch.float32, device=dev)
    pos = torch.empty((T, E), dtype=torch.int32, device=dev)
    back_p = torch.empty((T, k), dtype=torch.float32, device=dev)
    back_i = torch.empty((T, k), dtype=torch.int32, device=dev)
    if has_ffn:
        H, I = w.H, w.I
        hidden, w13, w2 = bf(inp["hidden"]), bf(inp["w13"]), bf(inp["w2"])
        act = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
        splits = moe.moe_ffn_down_splits(moe.MOE_BF16, T, H, I, E, k, decode)
        y = torch.empty((splits, T * k, H), dtype=torch.float32, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    # Route, the indices->multihot conversion of its output, the alignment and
    # the multihot->indices conversion of the maps run as one call
    # (moe_route_align_inverse; its launches are in config).
    phases = ["route_align_inverse"]
    ra_out = {"topk_w": topk_w, "topk_ids": topk_ids, "multihot": mh, "probs_in_multihot": pim,
              "position_map": pos, **aligned, "probs_indices": back_p,
              "ids_from_multihot": back_i}
    if grouped:  # group-limited selection (+ indices->multihot), then align + the inverse
        phases = ["route_grouped", "align_inverse"]
    ai_out = {**aligned, "probs_indices": back_p, "ids_from_multihot": back_i}
    # Decode: FC2 and the combine through one call (one launch where fused);
    # for the smallest batches the routing call and FC1 are one call as well.
    route_fc1 = has_ffn and decode and moe.moe_route_align_gate_up_fused(
        T, E, k, moe.MOE_BF16, decode, w.H, w.I)
    if route_fc1:
        phases = ["route_align_gate_up", "down_combine"]
    elif has_ffn and decode:
        phases += ["gate_up", "down_combine"]
    elif has_ffn:
        phases += ["gate_up", "down", "combine"]

    cur = {"logits": logits_draws[0]}

    def run_phase(name):
        if name == "route_align_inverse":
            moe.moe_route_align_inverse(cur["logits"], k, w.norm, out=ra_out, workspace=align_ws)
        elif name == "route_align_gate_up":
            moe.moe_route_align_gate_up(cur["logits"], k, hidden, w13, w.norm, decode=True,
                                        inverse=True, out=ra_out, act=act, workspace=align_ws)
        elif name == "route_grouped":
            moe.moe_route_grouped(cur["logits"], k, w.n_group, w.topk_group, w.method, bias_d,
                                  w.renorm, topk_w, topk_ids, multihot=(mh, pim, pos))
        elif name == "to_multihot":
            moe.moe_indices_to_multihot(topk_ids, topk_w, E, out=(mh, pim, pos))
        elif name == "align":
            moe.moe_align(topk_ids, E, aligned, align_ws)
        elif name == "align_inverse":
            moe.moe_align_inverse(topk_ids, E, pim, pos, ai_out, align_ws)
        elif name == "to_indices":
            moe.moe_multihot_to_indices(pim, pos, k, out=(back_p, back_i))
        elif name == "gate_up":
            moe.moe_ffn_gate_up(hidden, w13, aligned, k, decode, act)
        elif name == "down":
            moe.moe_ffn_down(act, w2, aligned, T, k, decode, y, splits)
        elif name == "combine":
            moe.moe_combine(y, topk_w, aligned["slot_to_sorted"], torch.bfloat16, out)
        elif name == "down_combine":
            moe.moe_ffn_down_combine(act, w2, topk_w, aligned, T, k, decode, y, out)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
          for _ in range(args.steps)]

    for it in range(args.warmup):
        cur["logits"] = logits_draws[it % draws]
        for ph in phases:
            run_phase(ph)
    torch.cuda.synchronize()

    n_distinct = []
    t0 = time.perf_counter()
    for s in range(args.steps):
        cur["logits"] = logits_draws[s % draws]
        if flush:
            flush_buf.fill_(float(s))
        ev[s][0].record()
        for i, ph in enumerate(phases):
            run_phase(ph)
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ms = None
    if use_graph:
        # The same step captured once and replayed: the input logits live in
        # one static buffer that each routing draw is copied into before its
        # replay (outside the timed events, like the cache flush).
        static_logits = torch.empty_like(logits_draws[0])
        static_logits.copy_(logits_draws[0])
        cur["logits"] = static_logits
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for ph in phases:
                run_phase(ph)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for ph in phases:
                run_phase(ph)
        for it in range(args.warmup):
            static_logits.copy_(logits_draws[it % draws])
            graph.replay()
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for st in range(args.steps):
            static_logits.copy_(logits_draws[st % draws])
            if flush:
                flush_buf.fill_(float(st))
            gev[st][0].record()
            graph.replay()
            gev[st][1].record()
        torch.cuda.synchronize()
        graph_ms = sum(a.elapsed_time(b) for a, b in gev) / args.steps

    if decode:
        # Distinct experts per routing draw (outside the timed region).
        for r in range(min(draws, args.steps)):
            cur["logits"] = logits_draws[r]
            run_phase("route_align_inverse")
            n_distinct.append(int((aligned["counts"] > 0).sum().item()))

    phase_ms = {ph: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) /
                args.steps for i, ph in enumerate(phases)}
    eager_ms = sum(phase_ms.values()) if flush else wall * 1e3 / args.steps
    # With a cache flush between steps the wall clock would include it, so the
    # step time is then the sum of the event-timed phases (or the graph
    # replay, bracketed by its own events).
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    value = T * 1e3 / ms_per_step
    # Median over the timed steps of the event-timed step (the graph replay,
    # or the first to the last phase event of an eager step).
    if graph_ms is not None:
        per_step = [a.elapsed_time(b) for a, b in gev]
    else:
        per_step = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)]
    median_ms = float(np.median(per_step))

    cfg = {"workload": w.name, "T": T, "E": E, "top_k": k,
           "routing_draws": draws, "cache_flush_between_steps": flush,
           "step_timing": "hip_graph_replay" if graph_ms is not None else "eager",
           "eager_ms_per_step": round(eager_ms, 4), "median_event_ms_per_step": round(median_ms, 4)}
    if grouped:
        cfg.update({"method": w.method, "n_group": w.n_group, "topk_group": w.topk_group,
                    "renormalize": w.renorm})
    else:
        cfg.update({"norm_topk_prob": w.norm,
                    "route_align_inverse_launches": (1 if T * k <= 512 else 2)
                    if moe.moe_route_align_fused(T, E, k) else 4})
    if has_ffn:
        cfg.update({"H": w.H, "I": w.I, "fc2_k_slices": splits})
        n_valid = int(aligned["offsets"][-1].item())
    roofline = None
    if has_ffn and not decode:
        # Algorithmic FLOPs of FC1 per launch: 2 * rows * (2I) * H.
        flops = 2.0 * n_valid * 2 * w.I * w.H
        achieved = flops / (phase_ms["gate_up"] * 1e-3) / 1e12
        roofline = {"kernel": "grouped_gemm_bf16_kernel<true, true, false, false, false> (FC1)",
                    "bound": "mfma",
                    "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic("gate_up", w.name)}
        layer_flops = 2.0 * n_valid * 3 * w.I * w.H
        cfg["layer_tflops_per_s"] = round(layer_flops / (ms_per_step * 1e-3) / 1e12, 1)
    elif has_ffn and decode:
        # Algorithmic bytes of decode FC1 per launch: the selected experts' w13
        # (mean over the routing draws) + the token rows + the activations.
        n_exp = sum(n_distinct) / len(n_distinct)
        nbytes = n_exp * 2 * w.I * w.H * 2 + T * w.H * 2 + n_valid * w.I * 2
        if route_fc1:
            # The same launch routes: + the logits, the weights and ids, the
            # multihot maps, the alignment and the inverse's reads and writes.
            nbytes += T * E * 4 + T * k * 8 + T * E * 9 + T * k * 12 + (2 * E + 1) * 4 + \
                T * E * 8 + T * k * 8
            achieved = nbytes / (phase_ms["route_align_gate_up"] * 1e-3) / 1e9
            kname, tkey = "decode_route_gate_up_kernel (route + align + FC1)", "decode_route_gate_up"
        else:
            achieved = nbytes / (phase_ms["gate_up"] * 1e-3) / 1e9
            kname, tkey = "decode_gate_up_kernel", "decode_gate_up"
        roofline = {"kernel": kname, "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(tkey, w.name)}
        cfg["distinct_experts_mean"] = round(n_exp, 2)
        cfg["route_align_gate_up_fused"] = bool(route_fc1)
        # FC2 + combine: the selected experts' w2, the activations and the
        # output (and y written and read back where the two are not fused).
        fused = moe.moe_ffn_down_combine_fused(moe.MOE_BF16, T, w.H, w.I, E, k, decode)
        dc_bytes = n_exp * w.H * w.I * 2 + n_valid * w.I * 2 + T * w.H * 2 + \
            (0 if fused else n_valid * w.H * 4 * 2)
        cfg["down_combine_fused"] = fused
        cfg["down_combine_hbm_gbs"] = round(dc_bytes / (phase_ms["down_combine"] * 1e-3) / 1e9,
                                            1)
        cfg["down_combine_traffic"] = measured_traffic("decode_down_combine", w.name)
        # The whole step against HBM: its algorithmic bytes (every selected
        # expert's w13 and w2 once, the logits, the routing and multihot
        # outputs, the inverse's reads and writes, the token rows and the
        # output) over the step time.
        step_bytes = n_exp * 3 * w.I * w.H * 2 + T * E * 4 + T * k * 8 + T * k * 12 + \
            T * E * 9 + T * E * 8 + T * k * 8 + T * w.H * 2 * 2
        cfg["step_hbm_gbs"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1)
        cfg["step_hbm_frac"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)

    if routing_only:
        # Algorithmic HBM bytes per phase: every input read once, every output
        # written once.
        nb = {"route_multihot": T * E * 4 + T * k * 8 + T * E * (1 + 4 + 4),
              "route_align_inverse": T * E * 4 + T * k * 8 + T * E * (1 + 4 + 4) + T * k * 12 +
              (2 * E + 1) * 4 + T * E * 8 + T * k * 8,
              "route_grouped": T * E * 4 + E * 4 + T * k * 8 + T * E * (1 + 4 + 4),
              "to_multihot": T * k * 8 + T * E * (1 + 4 + 4),
              "align": T * k * 4 + T * k * 12 + (2 * E + 1) * 4,
              "align_inverse": T * k * 4 + T * k * 12 + (2 * E + 1) * 4 + T * E * 8 + T * k * 8,
              "to_indices": T * E * 8 + T * k * 8}
        nb = {ph: nb[ph] for ph in phases}
        dom = max(phase_ms, key=phase_ms.get)
        names = {"route_multihot": "route_rows16_kernel (route + multihot)",
                 "route_align_inverse": "route_hist_kernel + align_scatter_kernel (route + "
                                        "multihot + align + inverse)",
                 "route_grouped": "route_grouped_rows16_kernel (selection + multihot)",
                 "to_multihot": "to_multihot kernel",
                 "align": "align_hist_kernel + align_scatter_kernel",
                 "align_inverse": "align_hist_kernel + align_scatter_kernel (with the inverse's "
                                  "blocks)",
                 "to_indices": "to_indices kernel"}
        achieved = nb[dom] / (phase_ms[dom] * 1e-3) / 1e9
        roofline = {"kernel": names[dom], "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(dom, w.name)}
        cfg["path_bytes"] = sum(nb.values())
        cfg["path_gbs_eager_phases"] = round(sum(nb.values()) / (sum(phase_ms.values()) * 1e-3) / 1e9, 1)
        cfg["path_gbs_step"] = round(sum(nb.values()) / (ms_per_step * 1e-3) / 1e9, 1)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generators, random-init weights)", "config": cfg,
        "roofline": roofline,
        "phase_ms": {k_: round(v, 4) for k_, v in phase_ms.items()},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
