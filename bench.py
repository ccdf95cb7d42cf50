#!/usr/bin/env python3
"""Sparse MoE FFN layer forward on one MI355X: tokens/s and roofline fractions.

A step is one moe_layer_forward call (route, dispatch, gate/up, down,
combine, and the shared expert where the workload has one) over one batch of
seeded synthetic tokens, with the inputs already resident in HBM. Steps
cycle over R slots, each with its own copy of the layer's weights (like a
stack of layers) and its own x batch, R chosen from the weight bytes a first
untimed call touches so that R of them span at least 2 GiB: the 256 MB
Infinity Cache cannot serve a repeat, so every step streams its weights
from HBM, and the routing changes from step to step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

With no --config it prints one JSON line for the largest single-GPU
workload, the skewed prefill layer (T=16384, d=2048, E=128, h=768, top-8),
carrying a sub-record for every other workload (tiny fp32, gemma-shaped,
decode at T = 1/4/16/64, shared-plus-routed, the sigmoid-scored layer and
4-bit decode) and measured achievable peaks. Stage durations come from HIP
events the library records on its own stream; ``roofline`` is the dominant
stage's algorithmic bytes (HBM-bound workloads) or FLOPs (MFMA-bound
workloads) per launch divided by its measured duration.
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
STAGE_KERNEL = {"route": ("route_kernel", "route_part_kernel"),
                "dispatch": ("scan_kernel", "route_finish_kernel", "route_tiny_kernel"),
                "gate_up": ("gemm_bf16_pers<0", "gemm_bf16_kernel<0", "gemm_small_kernel<0",
                            "gemm_small_q4_lds<0"),
                "down": ("gemm_bf16_pers<1", "gemm_bf16_kernel<1", "gemm_small_kernel<1",
                         "gemm_small_pers<1", "gemm_small_q4_lds<1", "down_combine_"),
                "combine": ("combine_",)}


FWD_SOURCES = ("expert_gemm.hip", "expert_gemm_small.hip", "route_dispatch.hip", "combine.hip",
               "moe_api.cpp", "tiny_route.h")
BWD_SOURCES = ("backward.hip", "route_dispatch.hip", "tiny_route.h")
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


def host_info():
    """CPU model and the BLAS library NumPy calls, with its thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
            threads = max(int(j.get("num_threads", 1)) for j in infos)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    return model, blas, int(threads)


def cpu_baseline(inp, budget_s=20.0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle.moe_oracle as O
    model, blas, threads = host_info()
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
    return {"value": Ts / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"first {Ts} of {spec.T} tokens of the same inputs, float64 NumPy oracle, "
                      f"median of {len(times)} run(s) of {med:.2f} s"}


# What each workload is judged against: its binding roof and the fraction of
# it the layer should reach (prefill-shaped: >= 50% of bf16 MFMA peak;
# decode-shaped and the HBM-bound gemma shape: >= 60% of HBM peak).
TARGET = {"gemma_upcycled": 0.60, "decode": 0.60, "decode_q4": 0.60,
          "skewed_prefill": 0.50, "shared_routed": 0.50, "small_moe_sigmoid": 0.50}

HEADLINE = "skewed_prefill"
SUBRECORDS = ("tiny_fp32", "gemma_upcycled", "decode@T1", "decode@T4", "decode@T16",
              "decode@T64", "shared_routed", "small_moe_sigmoid", "decode_q4@T1",
              "decode_q4@T64")

# at most this many weight copies (the tiny layer's 0.8 MB would need
# thousands; its time is launch latency either way)
MAX_SLOTS = 256
# spin-kernel cycles per traced step held ahead of the host's launches
# (about 0.1 ms per step at the shader clock)
HOLD_CYCLES_PER_STEP = 200_000

WNAMES = ("w_router", "b_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
          "w_shared_gate", "w_gate_sb", "w_up_sb", "w_down_sb")


def to_device(a):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.uint32:  # packed scale|bias words
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def touched_weight_bytes(spec, U):
    """Bytes of weights one call must read: the U touched routed experts, the
    router and the shared expert."""
    from mixture_experts_sparse_amd import roofline as R
    eb = R.Q4_BYTES_PER_WEIGHT if spec.expert_quant else spec.act_bytes
    n = U * 3.0 * spec.d * spec.h * eb + spec.E * spec.d * spec.act_bytes
    if spec.shared_h:
        n += 3.0 * spec.d * spec.shared_h * spec.act_bytes
    return n


def isolated_stage_us(call, steps, nstages=None):
    """Mean duration (us) of every stage of ``call(i, events)``, each timed in
    a pass of ``steps`` calls of its own whose event rows hold only that
    stage's two boundary events (the others NULL, which the library skips)."""
    import ctypes

    import numpy as np
    import torch

    import mixture_experts_sparse_amd.binding as B
    from mixture_experts_sparse_amd.hip_timing import StageEvents

    n = B.MOE_NUM_STAGES if nstages is None else nstages
    out = []
    for s in range(n):
        ev = StageEvents(steps, n)
        rows = []
        for i in range(steps):
            arr = (ctypes.c_void_p * (n + 1))()
            arr[s], arr[s + 1] = ev.row(i)[s], ev.row(i)[s + 1]
            rows.append(arr)
        torch.cuda.synchronize()
        torch.cuda._sleep(HOLD_CYCLES_PER_STEP * steps)
        for i in range(steps):
            call(i, rows[i])
        torch.cuda.synchronize()
        ev.hip.hipEventSynchronize(ev.row(steps - 1)[s + 1])
        out.append(float(np.mean([ev.elapsed_ms(ev.row(i)[s], ev.row(i)[s + 1])
                                  for i in range(steps)])) * 1e3)
        ev.destroy()
    return out


def measure_forward(name, steps, warmup, rotate_gib, inp=None, calibrate_copy_mib=0):
    """Times moe_layer_forward on one workload. Steps cycle over R slots, each
    with its own copy of the weights and its own x batch (copy 0: the
    workload's x; others: moe_inputs.rotation_x), R chosen from the touched
    weight bytes of a first untimed call so that R of them span at least
    ``rotate_gib`` GiB: the 256 MB Infinity Cache cannot serve a repeat.
    Returns (record, generated inputs)."""
    import numpy as np
    import torch

    import mixture_experts_sparse_amd.binding as B
    from mixture_experts_sparse_amd import roofline as R
    from mixture_experts_sparse_amd.hip_timing import StageEvents
    from moe_inputs import generate, spec_by_name
    from moe_inputs.generate import rotation_x

    spec = spec_by_name(name)
    base = name.split("@")[0]
    T = spec.T
    t0 = time.perf_counter()
    if inp is None:
        inp = generate(spec)
    log(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f} s")
    cfg = B.config_from_spec(spec)
    w0 = {n: to_device(inp.get(n)) for n in WNAMES}
    xs = [to_device(inp["x"][:T])]
    out = torch.empty((T, spec.d), dtype=xs[0].dtype, device="cuda")
    ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
    counts = torch.empty(spec.E, dtype=torch.int32, device="cuda")
    ws = B.alloc_workspace(cfg)
    B.layer_forward(cfg, w0, xs[0], out=out, ids=ids, counts=counts, ws=ws)
    torch.cuda.synchronize()
    U0 = int((counts.cpu().numpy() > 0).sum())
    nslots = max(2, math.ceil(rotate_gib * 2**30 / touched_weight_bytes(spec, U0)))
    capped = nslots > MAX_SLOTS  # only the launch-bound tiny layer gets here
    nslots = min(nslots, MAX_SLOTS)
    wsets = [w0] + [{n: (t.clone() if t is not None else None) for n, t in w0.items()}
                    for _ in range(nslots - 1)]
    wstructs = [B.weights_struct(w) for w in wsets]
    xs += [to_device(rotation_x(spec, i)) for i in range(1, nslots)]
    # touched experts of every slot (the routing changes with x)
    slot_U, slot_load = [], []
    for i in range(nslots):
        B.layer_forward(cfg, wstructs[i], xs[i], out=out, ids=ids, counts=counts, ws=ws)
        torch.cuda.synchronize()
        c = counts.cpu().numpy()
        slot_U.append(int((c > 0).sum()))
        slot_load.append(float(c.max() / max(c.mean(), 1e-9)))
    set_bytes = sum(t.numel() * t.element_size() for t in w0.values() if t is not None)
    log(f"[bench] {name}: {nslots} slots (weights {set_bytes / 2**20:.1f} MiB each, touched "
        f"{touched_weight_bytes(spec, U0) / 2**20:.1f} MiB per call), workspace "
        f"{ws.numel() / 2**20:.1f} MiB")

    def call(i, ev=None):
        j = i % nslots
        B.layer_forward(cfg, wstructs[j], xs[j], out=out, ids=ids, counts=counts, ws=ws,
                        stage_events=ev)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()

    # timed region: K untraced steps between two events on the launch stream
    outer = StageEvents(1, 1)
    hip = outer.hip
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    w_start = time.perf_counter()
    hip.hipEventRecord(outer.row(0)[0], stream)
    for i in range(steps):
        call(i)
    hip.hipEventRecord(outer.row(0)[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w_start
    hip.hipEventSynchronize(outer.row(0)[1])
    span_ms = outer.elapsed_ms(outer.row(0)[0], outer.row(0)[1])
    outer.destroy()
    ms_per_step = span_ms / steps
    log(f"[bench] {name}: {steps} steps, {ms_per_step * 1e3:.1f} us/step (events), "
        f"{wall / steps * 1e6:.1f} us/step (wall)")

    # stage durations: the same K steps again with an event at every stage
    # boundary (each event pair adds a few microseconds of its own)
    ev = StageEvents(steps)
    torch.cuda.synchronize()
    # a bounded spin kernel holds the stream while the host enqueues the
    # traced steps, so that no stage interval absorbs a host launch gap
    torch.cuda._sleep(HOLD_CYCLES_PER_STEP * steps)
    for i in range(steps):
        call(i, ev.row(i))
    torch.cuda.synchronize()
    stage = np.array(ev.stage_ms())  # [steps, stages]
    traced_ms = ev.span_ms() / steps
    ev.destroy()
    # each stage alone: K more steps with events at that stage's two
    # boundaries only, so no other event's overhead falls inside it
    iso_us = isolated_stage_us(call, steps)
    # every step on its own: an event pair around each of K more calls (the
    # stream held while they are enqueued), for the spread of step times
    pc = StageEvents(steps, 1)
    torch.cuda.synchronize()
    torch.cuda._sleep(HOLD_CYCLES_PER_STEP * steps)
    for i in range(steps):
        r = pc.row(i)
        hip.hipEventRecord(r[0], stream)
        call(i)
        hip.hipEventRecord(r[1], stream)
    torch.cuda.synchronize()
    step_us = np.array(pc.stage_ms())[:, 0] * 1e3
    pc.destroy()
    step_pct = {q: float(np.percentile(step_us, v)) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    if calibrate_copy_mib > 0:
        n = calibrate_copy_mib * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {calibrate_copy_mib} MiB done")
        del src, dst

    step_U = [slot_U[i % nslots] for i in range(steps)]
    Umean = float(np.mean(step_U))
    mean_stage_us = dict(zip(B.STAGE_NAMES, iso_us))
    bound = BOUND[base]
    dom = max(mean_stage_us, key=mean_stage_us.get)
    dwork = [stage_work(spec, U, T)[dom] for U in step_U]
    dbytes = float(np.mean([w[0] for w in dwork]))
    dflops = float(np.mean([w[1] for w in dwork]))
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
    roof["traffic"] = recorded_traffic(name, dom)
    roof["alg_bytes"] = dbytes
    roof["alg_flops"] = dflops
    roof["kernel"] = dom

    sec = ms_per_step * 1e-3
    eb = R.Q4_BYTES_PER_WEIGHT if spec.expert_quant else None
    lflops = R.layer_flops(T, spec.d, spec.E, spec.h, spec.k, spec.shared_h, spec.shared_gate)
    lbytes = float(np.mean([R.layer_bytes(T, spec.d, spec.E, spec.h, U, spec.act_bytes,
                                          spec.shared_h, spec.shared_gate,
                                          spec.router_bias is not None, eb) for U in step_U]))
    layer = {"mfma_frac": lflops / sec / R.PEAK_BF16_MFMA_FLOPS,
             "hbm_frac": lbytes / sec / R.PEAK_HBM_BYTES,
             "alg_flops": lflops, "alg_bytes": lbytes, "touched_experts_mean": Umean,
             "touched_experts_first_call": U0,
             "max_over_mean_load": float(np.mean(slot_load))}
    rec = {
        "workload": name, "tokens_per_s": T / sec, "ms_per_step": ms_per_step, "steps": steps,
        "warmup": warmup, "dtype": "bf16" if spec.dtype == 1 else "f32",
        "config": {"workload": name, "T": T, "d": spec.d, "E": spec.E, "h": spec.h,
                   "top_k": spec.k, "shared_h": spec.shared_h,
                   "gates": ["softmax over all", "softmax over the selected",
                             "sigmoid affinities, selection-only balance bias"][spec.mode]
                   + (" + renormalised" if spec.renormalize else ""),
                   "routed_weights": spec.expert_quant or "activation dtype",
                   "rotation_slots": nslots, "rotation_capped": capped, "x_rotates": True,
                   "touched_weight_bytes_first_call": touched_weight_bytes(spec, U0),
                   "parallelism": "single GPU"},
        "roofline": roof, "layer": layer, "stages_us": mean_stage_us,
        "traced_us_per_step": traced_ms * 1e3,
        "step_us_each": step_pct,
    }
    if base in TARGET:
        frac = layer["mfma_frac"] if bound == "mfma" else layer["hbm_frac"]
        rec["target"] = {"roof": bound, "layer_frac": frac, "needed": TARGET[base],
                         "met": bool(frac >= TARGET[base])}
    del wsets, wstructs, xs, w0, ws, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, inp


def achievable_peaks():
    """Measured ceilings for context beside the published peaks: a 1 GiB
    device-to-device copy (bytes read plus written over its time) and a
    library bf16 matrix product of 8192^3 (torch's GEMM)."""
    import torch
    from mixture_experts_sparse_amd.hip_timing import StageEvents
    ev = StageEvents(1, 1)
    hip = ev.hip
    stream = torch.cuda.current_stream().cuda_stream
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    hip.hipEventRecord(ev.row(0)[0], stream)
    for _ in range(10):
        dst.copy_(src)
    hip.hipEventRecord(ev.row(0)[1], stream)
    torch.cuda.synchronize()
    copy_s = ev.elapsed_ms(ev.row(0)[0], ev.row(0)[1]) * 1e-3 / 10
    del src, dst
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    hip.hipEventRecord(ev.row(0)[0], stream)
    for _ in range(10):
        a @ b
    hip.hipEventRecord(ev.row(0)[1], stream)
    torch.cuda.synchronize()
    mm_s = ev.elapsed_ms(ev.row(0)[0], ev.row(0)[1]) * 1e-3 / 10
    ev.destroy()
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": 2.0 * n / copy_s / 1e9,
            "bf16_gemm_8192_TFLOPs": 2.0 * 8192 ** 3 / mm_s / 1e12,
            "what": "1 GiB device copy (read + write bytes) and torch bf16 8192^3 matmul, "
                    "10 calls each, HIP events"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="one workload only (skewed_prefill, gemma_upcycled, shared_routed, "
                         "decode@T1/4/16/64, decode_q4@T1/..., small_moe_sigmoid, tiny_fp32); "
                         "default: the skewed_prefill headline plus a sub-record for every "
                         "other workload")
    ap.add_argument("--rotate-gib", type=float, default=2.0,
                    help="minimum bytes of touched weights cycled through between repeats")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subrecords", action="store_true")
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

    import torch
    torch.cuda.set_device(0)

    if args.which != "forward":
        run_other_pass(args)
        return

    name = args.config or HEADLINE
    rec, inp = measure_forward(name, args.steps, args.warmup, args.rotate_gib,
                               calibrate_copy_mib=args.calibrate_copy_mib)
    result = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "layer": rec["layer"],
        "target": rec.get("target"),
        "stages_us": rec["stages_us"],
        "traced_us_per_step": rec["traced_us_per_step"],
        "step_us_each": rec["step_us_each"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    del inp
    if args.config is None and not args.no_subrecords:
        subs = {}
        cache = {}
        for sub in SUBRECORDS:
            base = sub.split("@")[0]
            sub_inp = None
            if "@T" in sub:
                # the batch sizes of one decode workload share one draw
                if base not in cache:
                    cache.clear()
                    from moe_inputs import generate, spec_by_name
                    cache[base] = generate(spec_by_name(f"{base}@T64"))
                from moe_inputs import spec_by_name
                sp = spec_by_name(sub)
                sub_inp = dict(cache[base], spec=sp, x=cache[base]["x"][:sp.T])
            r, _ = measure_forward(sub, args.steps, args.warmup, args.rotate_gib, inp=sub_inp)
            subs[sub] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "roofline", "layer",
                                           "target", "stages_us", "step_us_each") if k in r}
            subs[sub]["rotation_slots"] = r["config"]["rotation_slots"]
        result["subrecords"] = subs
        result["achievable_peaks"] = achievable_peaks()
    print(json.dumps(result), flush=True)


def run_other_pass(args):
    """The backward or routing-statistics line for one workload (gemma by
    default): weight copies spanning --rotate-gib, one x."""
    import numpy as np
    import torch

    import mixture_experts_sparse_amd.binding as B
    from mixture_experts_sparse_amd import roofline as R
    from mixture_experts_sparse_amd.hip_timing import StageEvents
    from moe_inputs import generate, spec_by_name

    name = args.config or "gemma_upcycled"
    args.config = name
    spec = spec_by_name(name)
    inp = generate(spec)
    w0 = {n: to_device(inp.get(n)) for n in WNAMES}
    set_bytes = sum(t.numel() * t.element_size() for t in w0.values() if t is not None)
    nsets = max(1, math.ceil(args.rotate_gib * 2**30 / set_bytes))
    wsets = [w0] + [{n: (t.clone() if t is not None else None) for n, t in w0.items()}
                    for _ in range(nsets - 1)]
    wstructs = [B.weights_struct(w) for w in wsets]
    x = to_device(inp["x"])
    cfg = B.config_from_spec(spec)
    if args.which == "backward":
        run_backward(args, spec, inp, cfg, x, wstructs, nsets, B, R, StageEvents)
    else:
        run_stats(args, spec, inp, cfg, x, w0, B, R, StageEvents)


def cpu_baseline_backward(inp, dout, budget_s=20.0):
    """The oracle's backward, as it stands, on a bounded sample of tokens."""
    import oracle.moe_oracle as O
    model, blas, threads = host_info()
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
            "cpu_model": model, "blas": blas,
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
    torch.cuda._sleep(HOLD_CYCLES_PER_STEP * args.steps)  # as in the forward's traced loop
    for i in range(args.steps):
        B.layer_backward(cfg, wstructs[i % nsets], x, dout, grads=grads, ws=ws,
                         stage_events=ev.row(i))
    torch.cuda.synchronize()
    traced_ms = ev.span_ms() / args.steps
    ev.destroy()

    def bcall(i, row):
        B.layer_backward(cfg, wstructs[i % nsets], x, dout, grads=grads, ws=ws, stage_events=row)

    iso_us = isolated_stage_us(bcall, args.steps, B.MOE_NUM_BWD_STAGES)
    if args.calibrate_copy_mib > 0:
        src = torch.empty(args.calibrate_copy_mib * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {args.calibrate_copy_mib} MiB done")
        del src, dst
    mean_stage_us = dict(zip(B.BWD_STAGE_NAMES, iso_us))
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
