#!/usr/bin/env python3
"""Sparse MoE FFN layer forward on one MI355X: tokens/s and roofline fractions.

A step is one moe_layer_forward call (route, dispatch, gate/up, down,
combine, and the shared expert where the workload has one) over one batch of
seeded synthetic tokens, with the inputs already resident in HBM. Steps
rotate over R distinct copies of the layer's weights (like a stack of
layers), R chosen so that the copies span at least 2 GiB: the 256 MB
Infinity Cache cannot serve repeats, so every step streams its weights from
HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Prints one JSON line. Stage durations come from HIP events the library
records on its own stream inside the timed loop; ``roofline`` is the
dominant stage's algorithmic bytes (HBM-bound workloads) or FLOPs
(MFMA-bound workloads) per launch divided by its measured duration.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s on 1 GPU; % bf16 MFMA peak (prefill) / % HBM BW (decode)"

# Binding roofline of each workload (algorithmic intensity vs the 312.5
# FLOP/B ridge of 2.5 PFLOP/s bf16 over 8 TB/s).
BOUND = {"tiny_fp32": "alu", "gemma_upcycled": "hbm", "decode": "hbm",
         "skewed_prefill": "mfma", "shared_routed": "mfma", "small_moe_sigmoid": "mfma",
         "decode_q4": "hbm"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(spec, U, T):
    """Algorithmic (bytes, flops) of each stage of one layer call."""
    from mixture_experts_sparse_amd import roofline as R
    b = spec.act_bytes
    d, h, E, k, hs = spec.d, spec.h, spec.E, spec.k, spec.shared_h
    P = T * k
    eb = R.Q4_BYTES_PER_WEIGHT if spec.expert_quant else None
    route_b = (E * d + T * d) * b + (4 * E if spec.router_bias else 0) + (d * b if spec.shared_gate else 0)
    route_f = 2.0 * T * d * E + (2.0 * T * d if spec.shared_gate else 0)
    return {
        "route": (route_b, route_f),
        "dispatch": (0.0, 0.0),
        "gate_up": (R.gate_up_bytes(T, d, h, U, b, hs, eb), R.gate_up_flops(P, d, h, T, hs)),
        "down": (R.down_bytes(d, h, U, b, hs, eb), R.down_flops(P, d, h, T, hs)),
        "combine": (T * d * b, 0.0),
    }


# kernel-name prefixes of each stage's (first) kernel in a rocprofv3 record
STAGE_KERNEL = {"route": ("route_kernel", "route_part_kernel"), "dispatch": ("scan_kernel",),
                "gate_up": ("gemm_bf16_pers<0", "gemm_bf16_kernel<0", "gemm_small_kernel<0",
                            "gemm_small_q4_kernel<0"),
                "down": ("gemm_bf16_pers<1", "gemm_bf16_kernel<1", "gemm_small_kernel<1",
                         "gemm_small_pers<1", "gemm_small_q4_kernel<1"),
                "combine": ("combine_",)}


FWD_SOURCES = ("expert_gemm.hip", "route_dispatch.hip", "combine.hip")
BWD_SOURCES = ("backward.hip", "route_dispatch.hip")
# kernel-name prefixes of each backward stage's product
BWD_STAGE_KERNEL = {"d_hidden": ("bwd_gemm<1>",), "z": ("bwd_gemm<0>",),
                    "dw_down": ("bwd_gemm<2>",), "dw_gate_up": ("bwd_gemm<3>",),
                    "dx_rows": ("bwd_gemm<4>",), "dx_router": ("bwd_gemm<5>",),
                    "router_grad": ("router_bwd_kernel",), "route": ("route_kernel",)}


def kernel_sources_sha(files=FWD_SOURCES):
    import hashlib
    d = os.path.join(ROOT, "mixture_experts_sparse_amd", "csrc")
    src = b"".join(open(os.path.join(d, f), "rb").read() for f in files)
    return hashlib.sha256(src).hexdigest()[:16]


def recorded_traffic(workload, stage, stage_kernel=STAGE_KERNEL, files=FWD_SOURCES):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE record, or None when there is no record for this
    workload or the kernels have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernels_sha256_16") != kernel_sources_sha(files):
        return None
    for name, t in rec["per_launch"].items():
        if any(k in name for k in stage_kernel.get(stage, ())):
            return t["fetch_bytes"] + t["write_bytes"]
    return None


def cpu_baseline(inp, budget_s=20.0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle.moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    spec = inp["spec"]

    def run(Ts):
        sub = dict(inp)
        sub["x"] = inp["x"][:Ts]
        sub["spec"] = dataclasses.replace(spec, T=Ts)
        t0 = time.perf_counter()
        O.layer_forward(sub)
        return time.perf_counter() - t0

    Ts = min(spec.T, 512)
    t = run(Ts)
    # grow the sample towards ~1/3 of the budget per run, capped at the batch
    while Ts < spec.T and t < budget_s / 6:
        Ts = min(spec.T, Ts * 2)
        t = run(Ts)
    times = [t]
    while len(times) < 3 and sum(times) + t < budget_s:
        times.append(run(Ts))
    med = statistics.median(times)
    return {"value": Ts / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {Ts} of {spec.T} tokens of the same inputs, float64 NumPy oracle, "
                      f"median of {len(times)} run(s) of {med:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gemma_upcycled",
                    help="workload name (gemma_upcycled, skewed_prefill, shared_routed, "
                         "decode@T1/4/16/64, tiny_fp32)")
    ap.add_argument("--rotate-gib", type=float, default=2.0,
                    help="minimum bytes of distinct weight copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--pass", dest="which", choices=("forward", "backward", "stats"),
                    default="forward",
                    help="forward (the headline), the layer backward (gradients of "
                         "sum(out * dout), recomputing route and pre-activations), or the "
                         "routing statistics of the workload's router logits")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a reference kernel for scaling profiler byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the layer forward here runs on a single MI355X "
              "and has no multi-GPU path (--gpus must be 1).", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_sparse_amd.binding as B
    from mixture_experts_sparse_amd import roofline as R
    from mixture_experts_sparse_amd.hip_timing import StageEvents
    from moe_inputs import generate, spec_by_name

    spec = spec_by_name(args.config)
    base = args.config.split("@")[0]
    t0 = time.perf_counter()
    inp = generate(spec)
    log(f"[bench] generated {args.config} in {time.perf_counter() - t0:.1f} s")
    torch.cuda.set_device(0)

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        if a.dtype == np.uint32:  # packed scale|bias words
            return torch.from_numpy(a.view(np.int32)).cuda()
        return torch.from_numpy(a).cuda()

    wnames = ("w_router", "b_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
              "w_shared_gate", "w_gate_sb", "w_up_sb", "w_down_sb")
    w0 = {n: dev(inp.get(n)) for n in wnames}
    set_bytes = sum(t.numel() * t.element_size() for t in w0.values() if t is not None)
    nsets = max(1, math.ceil(args.rotate_gib * 2**30 / set_bytes))
    wsets = [w0] + [{n: (t.clone() if t is not None else None) for n, t in w0.items()}
                    for _ in range(nsets - 1)]
    wstructs = [B.weights_struct(w) for w in wsets]
    x = dev(inp["x"])
    cfg = B.config_from_spec(spec)
    T = spec.T
    if args.which == "backward":
        run_backward(args, spec, inp, cfg, x, wstructs, nsets, B, R, StageEvents)
        return
    if args.which == "stats":
        run_stats(args, spec, inp, cfg, x, w0, B, R, StageEvents)
        return
    out = torch.empty((T, spec.d), dtype=x.dtype, device="cuda")
    ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
    counts = torch.empty(spec.E, dtype=torch.int32, device="cuda")
    ws = B.alloc_workspace(cfg)
    log(f"[bench] {nsets} weight copies of {set_bytes / 2**20:.1f} MiB, workspace "
        f"{ws.numel() / 2**20:.1f} MiB")

    for i in range(args.warmup):
        B.layer_forward(cfg, wstructs[i % nsets], x, out=out, ids=ids, counts=counts, ws=ws)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # Timed region: K untraced steps between two events on the launch stream.
    outer = StageEvents(1)
    hip = outer.hip
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    w_start = time.perf_counter()
    hip.hipEventRecord(outer.row(0)[0], stream)
    for i in range(args.steps):
        B.layer_forward(cfg, wstructs[i % nsets], x, out=out, ids=ids, counts=counts, ws=ws)
    hip.hipEventRecord(outer.row(0)[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w_start
    hip.hipEventSynchronize(outer.row(0)[1])
    span_ms = outer.elapsed_ms(outer.row(0)[0], outer.row(0)[1])
    outer.destroy()
    ms_per_step = span_ms / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (events), "
        f"{wall / args.steps * 1e6:.1f} us/step (wall)")

    # Stage durations: the same K steps again, with the library recording an
    # event at every stage boundary on its stream (each event pair adds a
    # few microseconds of its own, so these are upper bounds).
    ev = StageEvents(args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        B.layer_forward(cfg, wstructs[i % nsets], x, out=out, ids=ids, counts=counts, ws=ws,
                        stage_events=ev.row(i))
    torch.cuda.synchronize()
    stage = np.array(ev.stage_ms())  # [steps, stages]
    traced_ms = ev.span_ms() / args.steps
    ev.destroy()
    log(f"[bench] traced steps: {traced_ms * 1e3:.1f} us/step")

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {args.calibrate_copy_mib} MiB done")
        del src, dst

    cnt = counts.cpu().numpy()
    U = int((cnt > 0).sum())
    mean_stage_us = {n: float(stage[:, i].mean() * 1e3) for i, n in enumerate(B.STAGE_NAMES)}
    work = stage_work(spec, U, T)
    bound = BOUND[base]
    dom = max(mean_stage_us, key=mean_stage_us.get)
    dbytes, dflops = work[dom]
    dsec = mean_stage_us[dom] * 1e-6
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": dflops / dsec / 1e12,
                "peak": R.PEAK_BF16_MFMA_FLOPS / 1e12, "unit": "TFLOP/s"}
    elif bound == "alu":
        roof = {"bound": "alu", "achieved": dflops / dsec / 1e12,
                "peak": R.PEAK_FP32_VALU_FLOPS / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": dbytes / dsec / 1e9,
                "peak": R.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(args.config, dom)
    roof["alg_bytes"] = dbytes
    roof["kernel"] = dom

    sec = ms_per_step * 1e-3
    lflops = R.layer_flops(T, spec.d, spec.E, spec.h, spec.k, spec.shared_h, spec.shared_gate)
    lbytes = R.layer_bytes(T, spec.d, spec.E, spec.h, U, spec.act_bytes, spec.shared_h,
                           spec.shared_gate, spec.router_bias is not None,
                           R.Q4_BYTES_PER_WEIGHT if spec.expert_quant else None)
    result = {
        "metric": METRIC,
        "value": T / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": args.config, "T": T, "d": spec.d, "E": spec.E, "h": spec.h,
                   "top_k": spec.k, "shared_h": spec.shared_h,
                   "gates": ["softmax over all", "softmax over the selected",
                             "sigmoid affinities, selection-only balance bias"][spec.mode]
                   + (" + renormalised" if spec.renormalize else ""),
                   "routed_weights": spec.expert_quant or "activation dtype",
                   "weight_copies": nsets, "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"mfma_frac": lflops / sec / R.PEAK_BF16_MFMA_FLOPS,
                  "hbm_frac": lbytes / sec / R.PEAK_HBM_BYTES,
                  "alg_flops": lflops, "alg_bytes": lbytes, "touched_experts": U,
                  "max_over_mean_load": float(cnt.max() / max(cnt.mean(), 1e-9))},
        "stages_us": mean_stage_us,
        "traced_us_per_step": traced_ms * 1e3,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


def cpu_baseline_backward(inp, dout, budget_s=20.0):
    """The oracle's backward, as it stands, on a bounded sample of tokens."""
    import oracle.moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    spec = inp["spec"]

    def run(Ts):
        sub = dict(inp)
        sub["x"] = inp["x"][:Ts]
        sub["spec"] = dataclasses.replace(spec, T=Ts)
        t0 = time.perf_counter()
        O.layer_backward(sub, dout[:Ts])
        return time.perf_counter() - t0

    Ts = min(spec.T, 256)
    t = run(Ts)
    while Ts < spec.T and t < budget_s / 6:
        Ts = min(spec.T, Ts * 2)
        t = run(Ts)
    times = [t]
    while len(times) < 3 and sum(times) + t < budget_s:
        times.append(run(Ts))
    med = statistics.median(times)
    return {"value": Ts / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {Ts} of {spec.T} tokens of the same inputs, float64 NumPy oracle "
                      f"backward, median of {len(times)} run(s) of {med:.2f} s"}


def run_backward(args, spec, inp, cfg, x, wstructs, nsets, B, R, StageEvents):
    """The layer backward: K timed moe_layer_backward calls (rotating weight
    copies), then K traced calls for the stage durations."""
    import numpy as np
    import torch
    from moe_inputs.generate import bf16_bits_from_f32
    if spec.dtype != 1:
        print("the layer backward runs on bf16 layers only", file=sys.stderr, flush=True)
        sys.exit(2)
    T = spec.T
    rng = np.random.default_rng(1234)
    dout_bits = bf16_bits_from_f32(rng.standard_normal((T, spec.d)).astype(np.float32))
    dout = torch.from_numpy(dout_bits.view(np.int16)).cuda().view(torch.bfloat16)
    ws = B.alloc_workspace(cfg, B.MOE_ENTRY_LAYER_BACKWARD)
    grads = B.layer_backward(cfg, wstructs[0], x, dout, ws=ws)
    log(f"[bench] backward workspace {ws.numel() / 2**20:.1f} MiB")
    for i in range(args.warmup):
        B.layer_backward(cfg, wstructs[i % nsets], x, dout, grads=grads, ws=ws)
    torch.cuda.synchronize()
    outer = StageEvents(1, 1)
    hip = outer.hip
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    hip.hipEventRecord(outer.row(0)[0], stream)
    for i in range(args.steps):
        B.layer_backward(cfg, wstructs[i % nsets], x, dout, grads=grads, ws=ws)
    hip.hipEventRecord(outer.row(0)[1], stream)
    torch.cuda.synchronize()
    hip.hipEventSynchronize(outer.row(0)[1])
    ms_per_step = outer.elapsed_ms(outer.row(0)[0], outer.row(0)[1]) / args.steps
    outer.destroy()
    log(f"[bench] backward: timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")
    ev = StageEvents(args.steps, B.MOE_NUM_BWD_STAGES)
    torch.cuda.synchronize()
    for i in range(args.steps):
        B.layer_backward(cfg, wstructs[i % nsets], x, dout, grads=grads, ws=ws,
                         stage_events=ev.row(i))
    torch.cuda.synchronize()
    stage = np.array(ev.stage_ms())
    traced_ms = ev.span_ms() / args.steps
    ev.destroy()
    if args.calibrate_copy_mib > 0:
        src = torch.empty(args.calibrate_copy_mib * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {args.calibrate_copy_mib} MiB done")
        del src, dst
    mean_stage_us = {n: float(stage[:, i].mean() * 1e3) for i, n in enumerate(B.BWD_STAGE_NAMES)}
    flops = R.backward_stage_flops(T, spec.d, spec.E, spec.h, spec.k, spec.shared_h,
                                   spec.shared_gate)
    nbytes = R.backward_stage_bytes(T, spec.d, spec.E, spec.h, spec.k, spec.shared_h)
    dom = max(mean_stage_us, key=mean_stage_us.get)
    dsec = mean_stage_us[dom] * 1e-6
    # the dominant stage against the roof its own work hits first: MFMA when
    # its FLOPs take longer at the bf16 peak than its bytes at the HBM peak
    if flops[dom] / R.PEAK_BF16_MFMA_FLOPS >= nbytes[dom] / R.PEAK_HBM_BYTES:
        roof = {"bound": "mfma", "achieved": flops[dom] / dsec / 1e12,
                "peak": R.PEAK_BF16_MFMA_FLOPS / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes[dom] / dsec / 1e9,
                "peak": R.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"],
                 "traffic": recorded_traffic(f"{args.config} backward", dom, BWD_STAGE_KERNEL,
                                             BWD_SOURCES),
                 "alg_flops": flops[dom], "alg_bytes": nbytes[dom], "kernel": dom})
    total = sum(flops.values())
    sec = ms_per_step * 1e-3
    result = {
        "metric": "MoE layer bwd tokens/s on 1 GPU (gradients of sum(out*dout), route and "
                  "pre-activations recomputed); dominant stage vs its roof",
        "value": T / sec, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config} backward", "T": T, "d": spec.d, "E": spec.E,
                   "h": spec.h, "top_k": spec.k, "shared_h": spec.shared_h,
                   "weight_copies": nsets, "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"mfma_frac": total / sec / R.PEAK_BF16_MFMA_FLOPS, "alg_flops": total},
        "stages_us": mean_stage_us,
        "traced_us_per_step": traced_ms * 1e3,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle backward baseline")
        result["cpu_baseline"] = cpu_baseline_backward(inp, dout_bits, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


def cpu_baseline_stats(inp, counts, budget_s=20.0):
    """The oracle's routing statistics, as they stand, on a bounded sample of
    tokens (router logits from the oracle's own router, not timed)."""
    import oracle.moe_oracle as O
    spec = inp["spec"]
    bias = None if spec.mode == O.SIGMOID else inp.get("b_router")
    L = O.router_logits(inp["x"], inp["w_router"], bias)

    def run(Ts):
        t0 = time.perf_counter()
        O.routing_stats(L[:Ts], counts, spec.k, spec.mode, 0.01)
        return time.perf_counter() - t0

    Ts = min(spec.T, 256)
    t = run(Ts)
    while Ts < spec.T and t < budget_s / 6:
        Ts = min(spec.T, Ts * 2)
        t = run(Ts)
    times = [t]
    while len(times) < 3 and sum(times) + t < budget_s:
        times.append(run(Ts))
    med = statistics.median(times)
    return {"value": Ts / med, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {Ts} of {spec.T} tokens' router logits, float64 NumPy oracle "
                      f"routing_stats, median of {len(times)} run(s) of {med:.3f} s"}


def run_stats(args, spec, inp, cfg, x, w0, B, R, StageEvents):
    """Routing statistics over the workload's router logits (moe_route's
    float32 output) and moe_dispatch's counts: K calls queued behind a long
    matrix product, so the event span is device time, not launch rate."""
    import torch
    T, E = spec.T, spec.E
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids, _ = B.route(cfg, x, w0["w_router"], w0["b_router"], logits=logits)
    counts, _, _, _ = B.dispatch(cfg, ids)
    ws = B.alloc_workspace(cfg, B.MOE_ENTRY_ROUTING_STATS)
    outs = (torch.empty(E, dtype=torch.float32, device="cuda"),
            torch.empty(E, dtype=torch.float32, device="cuda"),
            torch.empty(4, dtype=torch.float32, device="cuda"))
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        B.routing_stats(cfg, logits, counts, ws=ws, outs=outs)
    a = torch.ones((8192, 8192), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    ev = StageEvents(1, 1)
    hip = ev.hip
    for _ in range(8):  # keeps the device busy while the K calls are queued
        a @ a
    hip.hipEventRecord(ev.row(0)[0], stream)
    for _ in range(args.steps):
        B.routing_stats(cfg, logits, counts, ws=ws, outs=outs)
    hip.hipEventRecord(ev.row(0)[1], stream)
    torch.cuda.synchronize()
    hip.hipEventSynchronize(ev.row(0)[1])
    us = ev.elapsed_ms(ev.row(0)[0], ev.row(0)[1]) * 1e3 / args.steps
    ev.destroy()
    log(f"[bench] routing stats: {us:.2f} us/call over {args.steps} queued calls")
    nbytes = R.routing_stats_bytes(T, E)
    roof = {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9,
            "peak": R.PEAK_HBM_BYTES / 1e9, "unit": "GB/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": None,
                 "alg_bytes": nbytes, "kernel": "routing_stats (both kernels)"})
    result = {
        "metric": "MoE routing statistics tokens/s on 1 GPU (token share, mean router "
                  "probability, router entropy, load-balance term)",
        "value": T / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config} routing statistics", "T": T, "E": E,
                   "top_k": spec.k, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle routing statistics")
        result["cpu_baseline"] = cpu_baseline_stats(inp, counts.cpu().numpy(), args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
