#!/usr/bin/env python3
"""Throughput of the GTR gated-linear-attention forward pass on one MI355X.

One step = every call of the chosen workload (e.g. the four scan directions of
a 4-layer round), each on its own seeded inputs already resident in HBM.
Steps are captured once in a HIP graph and replayed; the timed region is K
replays bracketed by device synchronisation, timed with HIP events on the
replay stream.  Prints one JSON line.

  value        tokens/s = sum over the step's calls of B*H*N, per second
  roofline     the dominant kernel's algorithmic bytes per launch over its
               average duration (HIP events around each launch, eager, on the
               launch stream), against 8 TB/s HBM
  cpu_baseline the fp64 oracle on the host cores, on the same step's inputs
  cold         the same step on copies of its tensors used in turn, so that
               more than 512 MB is touched between two uses of one copy (no
               input is still in the 256 MB Infinity Cache when read again);
               value is the warm figure above
  long_sequence  the default run (1,600 tokens) also times the 16,384-token
               round the same way: the metric is quoted at both lengths
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2,
                    help="1..5; default 2 = 40x40 grid, fp16, B1 H6, four directions")
    ap.add_argument("--chunks-per-segment", type=int, default=0)
    ap.add_argument("--path", choices=["auto", "fused", "split"], default="auto")
    ap.add_argument("--head-dims", type=int, nargs=2, metavar=("D_K", "D_V"), default=None,
                    help="run the workload with these head dims instead of 64 x 64")
    ap.add_argument("--directions", type=int, nargs="+", default=None, choices=[0, 1, 2, 3],
                    help="run the workload's grid in these scan directions instead of its own "
                         "(0 L->R, 1 R->L, 2 T->B, 3 B->T), one call each")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-sequence", action="store_true",
                    help="skip the 16,384-token round the default run also reports")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--profile-steps", type=int, default=50)
    ap.add_argument("--op", choices=["gla", "bwd", "swiglu"], default="gla",
                    help="gla: the attention forward (default); bwd: its backward pass; "
                         "swiglu: the Spatial SwiGLU block")
    ap.add_argument("--swiglu-workload", type=int, default=1,
                    help="1 = 40x40 grid, C 384, F 1024; 2 = 128x128 grid, C 1024, F 2752 (fp16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes ten times (the reference "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE readings) and exit")
    return ap.parse_args()


def copy_calibration(n_bytes: int) -> None:
    import torch
    src = torch.ones(n_bytes // 2, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n_bytes, "launches": 10}), flush=True)


def measured_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rows = json.load(f)
    for r in rows:
        if r.get("kernel") == kernel and r.get("workload") == workload and r.get("source") == digest:
            return r.get("hbm_bytes_per_launch")
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this operator is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.op == "swiglu":
        swiglu_main(args)
        return
    if args.op == "bwd":
        bwd_main(args)
        return

    import torch

    import gla_inputs
    import recurrent_vision_backbone_chunkwise_amd as gla

    if not os.path.exists(gla.LIB_PATH):
        from recurrent_vision_backbone_chunkwise_amd import build as hip_build
        hip_build.build()
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    w = gla_inputs.workload(args.workload)
    if args.head_dims and tuple(args.head_dims) != (w.d_k, w.d_v):
        dk, dv = args.head_dims
        w = dataclasses.replace(w, d_k=dk, d_v=dv, name=f"{w.name}_dk{dk}_dv{dv}")
    if args.directions and tuple(args.directions) != tuple(w.directions):
        names = "".join(gla_inputs.DIR_NAMES[d].replace("->", "").lower() for d in args.directions)
        w = dataclasses.replace(w, directions=tuple(args.directions), name=f"{w.name}_dirs_{names}")
    path = {"auto": 0, "fused": 1, "split": 2}[args.path]
    m = measure_gla(args, w, path, args.chunks_per_segment, args.steps, with_cold=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, m["cpu_inputs"], args.cpu_seconds)

    # The metric is quoted at 1.6K and at 16K tokens: the default run also times the
    # 16,384-token round (workload 5) the same way and reports it beside the main figure.
    long_seq = None
    if args.workload == 2 and not args.head_dims and not args.directions and path == 0 and not args.no_long_sequence:
        w5 = gla_inputs.workload(5)
        m5 = measure_gla(args, w5, 0, 0, min(args.steps, 100), with_cold=False)
        long_seq = {"workload": w5.name, "value": round(m5["value"], 1), "unit": "tokens/s",
                    "ms_per_step": round(m5["ms_per_step"], 6), "steps": min(args.steps, 100),
                    "tokens_per_step": m5["tokens_per_step"],
                    "roofline": {k: m5["roofline"][k] for k in ("bound", "kernel", "achieved", "peak",
                                                                  "unit", "frac", "traffic", "kernel_frac",
                                                                  "call_achieved", "call_frac")}}

    plan = m["plan"]
    line = {
        "metric": "GLA fwd tokens/sec (B*H*N), one MI355X",
        "value": round(m["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "grid": [w.grid_h, w.grid_w], "n_tok": w.n_tok,
            "d_k": w.d_k, "d_v": w.d_v, "io_dtype": w.dtype, "gate": w.gate,
            "directions": [gla_inputs.DIR_NAMES[d] for d in w.directions],
            "tokens_per_step": m["tokens_per_step"], "chunks_per_segment": plan["seg_len"],
            "segments_per_sequence": plan["n_seg"], "kernels": "fused" if plan["fused"] else "split",
            "timing": "eager" if args.eager else "hip graph replay", "wall_ms": round(m["wall_ms"], 3),
            "accumulate": "f32",
        },
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
        "cold": m["cold"],
        "long_sequence": long_seq,
    }
    print(json.dumps(line), flush=True)


def measure_gla(args, w, path, cps, steps, with_cold):
    """Times `steps` replays of the workload's round (one HIP graph, HIP events on its stream),
    then the per-kernel durations of eager launches, and derives the dominant kernel's roofline."""
    import torch

    import gla_inputs
    import recurrent_vision_backbone_chunkwise_amd as gla

    dev = torch.device("cuda:0")
    plan = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, cps, path, w.d_k, w.d_v)
    cpu_inputs = [gla_inputs.workload_inputs(w, layer) for layer in range(len(w.directions))]
    inputs = [[x.to(dev) for x in ins] for ins in cpu_inputs]
    outs = [torch.empty_like(ins[2]) for ins in inputs]
    tokens_per_call = w.B * w.H * w.n_tok
    tokens_per_step = tokens_per_call * len(w.directions)
    elt = 4 if w.dtype == "f32" else 2

    stream = torch.cuda.Stream()

    def step():
        for (q, k, v, g), d, o in zip(inputs, w.directions, outs):
            gla.gtr_gla_fwd_ex(q, k, v, g, o, d, chunks_per_segment=cps, path=path, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(steps):
            if graph is not None:
                graph.replay()
            else:
                step()
        stop.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = start.elapsed_time(stop) / steps
    value = tokens_per_step / (ms_per_step * 1e-3)

    cold = None
    if with_cold:
        cold = cold_round(args, w, inputs, outs, cps, path, stream, tokens_per_step, graph is not None)

    # per-kernel durations: HIP events around every launch, eager, same stream
    gla.gtr_gla_profile_begin()
    with torch.cuda.stream(stream):
        for _ in range(args.profile_steps):
            step()
    prof = gla.gtr_gla_profile_end()
    torch.cuda.synchronize()
    kern = {name: {"avg_us": 1e3 * ms / n, "launches_per_step": n / args.profile_steps}
            for name, (ms, n) in prof.items() if n > 0}
    dominant = max(kern, key=lambda n: kern[n]["avg_us"] * kern[n]["launches_per_step"])
    seg_len, n_seg = plan["seg_len"], plan["n_seg"]
    # algorithmic bytes per launch of each kernel (what it must move at minimum)
    alg_bytes = {
        "gla_fused": tokens_per_call * (3 * w.d_k + 2 * w.d_v) * elt,
        "gla_seg_out": tokens_per_call * (3 * w.d_k + 2 * w.d_v) * elt,
        "gla_seg_state": w.B * w.H * min(w.n_tok, (n_seg - 1) * seg_len * 64) * (2 * w.d_k + w.d_v) * elt,
        "gla_seg_scan": w.B * w.H * n_seg * w.d_k * w.d_v * 4 * 2,
    }
    avg_s = kern[dominant]["avg_us"] * 1e-6
    achieved = alg_bytes[dominant] / avg_s / 1e9
    from recurrent_vision_backbone_chunkwise_amd.build import source_digest
    digest = source_digest()
    traffic = measured_traffic(dominant, w.name, digest)
    call_gbs = value * (3 * w.d_k + 2 * w.d_v) * elt / 1e9
    # frac: the dominant kernel (its algorithmic bytes per launch over its average launch);
    # call_frac: whole calls (every kernel of the step, launch gaps included) over the step time
    roofline = {
        "bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel_frac": round(achieved / HBM_PEAK_GBS, 4),
        "call_achieved": round(call_gbs, 1), "call_frac": round(call_gbs / HBM_PEAK_GBS, 4),
        "alg_bytes_per_launch": alg_bytes[dominant], "avg_launch_us": round(kern[dominant]["avg_us"], 3),
        "kernels": {n: {"avg_us": round(v["avg_us"], 3), "per_step": v["launches_per_step"]}
                    for n, v in kern.items()},
        "source": digest,
    }
    result = {"value": value, "ms_per_step": ms_per_step, "wall_ms": wall_ms, "cold": cold,
              "roofline": roofline, "plan": plan, "tokens_per_step": tokens_per_step,
              "cpu_inputs": cpu_inputs}
    del graph, inputs, outs
    torch.cuda.synchronize()
    return result


COLD_BYTES = 512 << 20  # twice the 256 MB Infinity Cache


def cold_round(args, w, inputs, outs, cps, path, stream, tokens_per_step, use_graph):
    """The same round, timed the same way, on copies of its tensors at other addresses, used in
    turn, so that more than COLD_BYTES are touched between two uses of one copy and no input is
    still cached when it is read again.  A round that alone exceeds COLD_BYTES is its own copy."""
    import torch

    import recurrent_vision_backbone_chunkwise_amd as gla

    round_bytes = sum(t.numel() * t.element_size() for ins in inputs for t in ins)
    round_bytes += sum(o.numel() * o.element_size() for o in outs)
    n_sets = max(1, -(-COLD_BYTES // round_bytes))
    sets = [(inputs, outs)] + [([[t.clone() for t in ins] for ins in inputs],
                                [torch.empty_like(o) for o in outs]) for _ in range(n_sets - 1)]

    def step(ins_set, out_set):
        for (q, k, v, g), d, o in zip(ins_set, w.directions, out_set):
            gla.gtr_gla_fwd_ex(q, k, v, g, o, d, chunks_per_segment=cps, path=path, stream=stream)

    graphs = []
    with torch.cuda.stream(stream):
        for ins_set, out_set in sets:
            step(ins_set, out_set)
    torch.cuda.synchronize()
    if use_graph:
        for ins_set, out_set in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                step(ins_set, out_set)
            graphs.append(gr)
        for gr in graphs:
            gr.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for i in range(args.steps):
            if use_graph:
                graphs[i % n_sets].replay()
            else:
                step(*sets[i % n_sets])
        stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    del graphs, sets
    return {"value": round(tokens_per_step / (ms * 1e-3), 1), "ms_per_step": round(ms, 6),
            "copies": n_sets, "bytes_between_reuse": n_sets * round_bytes}


def cpu_baseline(w, cpu_inputs, budget_s):
    """The fp64 oracle, as it is, on the step's own inputs.  The step's calls are independent
    (each direction has its own inputs), so they run concurrently, each parallel over its B*H
    sequences with an equal share of the host's cores; the step is repeated until about
    budget_s of wall time."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    host = len(os.sched_getaffinity(0))
    n_calls = len(w.directions)
    per_call = max(1, host // n_calls)
    used = [0] * n_calls

    def run(i):
        q, k, v, g = cpu_inputs[i]
        _, used[i] = oracle.gla_forward(q, k, v, g, w.directions[i], n_threads=per_call, return_threads=True)

    reps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(n_calls) as ex:
        while True:
            list(ex.map(run, range(n_calls)))
            reps += 1
            t = time.perf_counter() - t0
            if t >= budget_s or reps >= 1000:
                break
    tokens = reps * n_calls * w.B * w.H * w.n_tok
    return {"value": round(tokens / t, 1), "unit": "tokens/s", "cores": sum(used), "host_cores": host,
            "kind": "oracle",
            "sample": f"the full step ({n_calls} calls of {w.name}, run concurrently, each on up to "
                      f"{per_call} threads) x {reps} repetitions, {t:.1f} s wall, fp64 token-by-token "
                      f"recurrence"}


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # MI355X dense


def bwd_main(args):
    """One step = the backward pass of every call of the workload's round (dout seeded, inputs and
    gradients resident in HBM)."""
    import torch

    import gla_inputs
    import recurrent_vision_backbone_chunkwise_amd as gla

    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    w = gla_inputs.workload(args.workload)
    if args.head_dims and tuple(args.head_dims) != (w.d_k, w.d_v):
        dk, dv = args.head_dims
        w = dataclasses.replace(w, d_k=dk, d_v=dv, name=f"{w.name}_dk{dk}_dv{dv}")
    cpu_in = [gla_inputs.workload_inputs(w, layer) for layer in range(len(w.directions))]
    douts = [gla_inputs.make_output_grad(ins[2].shape, w.dtype, seed=9000 + i) for i, ins in enumerate(cpu_in)]
    ins = [[t.to("cuda:0") for t in x] + [d.to("cuda:0")] for x, d in zip(cpu_in, douts)]
    grads = [[torch.empty_like(x[0]), torch.empty_like(x[1]), torch.empty_like(x[2]), torch.empty_like(x[3])]
             for x in ins]
    stream = torch.cuda.Stream()

    def step():
        for (q, k, v, g, do), (dq, dk, dv, dg), d in zip(ins, grads, w.directions):
            gla.gtr_gla_bwd(q, k, v, g, do, dq, dk, dv, dg, d, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        graph.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(args.steps):
            graph.replay() if graph is not None else step()
        stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    tokens_per_call = w.B * w.H * w.n_tok
    tokens = tokens_per_call * len(w.directions)
    value = tokens / (ms_per_step * 1e-3)

    gla.gtr_gla_profile_begin()
    with torch.cuda.stream(stream):
        for _ in range(args.profile_steps):
            step()
    prof = gla.gtr_gla_profile_end()
    torch.cuda.synchronize()
    kern = {n: (1e3 * ms / c, c / args.profile_steps) for n, (ms, c) in prof.items() if c > 0}
    dominant = max(kern, key=lambda n: kern[n][0] * kern[n][1])
    elt = 4 if w.dtype == "f32" else 2
    dk, dv = w.d_k, w.d_v
    chunks = w.B * w.H * ((w.n_tok + 63) // 64)
    # the chunk kernel: reads kop, gates, a, b and writes its output (algorithmic bytes); its
    # contractions are the lower-triangle scores (fp16 MFMA for 16-bit I/O, whose inputs are exact
    # in fp16; fp32 otherwise), the state term and the intra-chunk sum (fp32 MFMA).  Its MFMA peak
    # is the rate that does this mix in the least time.
    bytes_dqk = tokens_per_call * (3 * dk + 2 * dv) * elt
    flops_scores = chunks * 2 * 64 * 64 * dv * 10 / 16
    flops_rest = chunks * (2 * 64 * dk * dv + 2 * 64 * 32 * dk)
    flops_dqk = flops_scores + flops_rest
    score_peak = MFMA_PEAK_TFLOPS["f32" if w.dtype == "f32" else "f16"]
    us = kern["gla_bwd_dqk"][0]
    t_hbm = bytes_dqk / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_scores / (score_peak * 1e12) + flops_rest / (MFMA_PEAK_TFLOPS["f32"] * 1e12)
    if t_mfma > t_hbm:
        rl = {"bound": "mfma", "achieved": flops_dqk / (us * 1e-6) / 1e12,
              "peak": round(flops_dqk / t_mfma / 1e12, 1), "unit": "TFLOP/s",
              "peak_mix": f"scores at {score_peak} TFLOP/s, the rest at {MFMA_PEAK_TFLOPS['f32']}"}
    else:
        rl = {"bound": "hbm", "achieved": bytes_dqk / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    rl["frac"] = round(rl["achieved"] / rl["peak"], 4)
    rl["achieved"] = round(rl["achieved"], 1)
    roofline = {**rl, "kernel": "gla_bwd_dqk", "traffic": None, "dominant_kernel": dominant,
                "kernels": {n: {"avg_us": round(t, 3), "per_step": c} for n, (t, c) in kern.items()}}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0, reps, threads = time.perf_counter(), 0, 1
        while True:
            for x, d, di in zip(cpu_in, douts, w.directions):
                oracle.gla_backward(*x, d, di)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 100:
                break
        t = time.perf_counter() - t0
        cpu = {"value": round(reps * tokens / t, 1), "unit": "tokens/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"the full step ({len(w.directions)} calls, {w.name}) x {reps}, {t:.1f} s, "
                         "fp64 chain rule token by token"}
    line = {
        "metric": "GLA backward tokens/sec (B*H*N), one MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if w.dtype == "f32" else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "grid": [w.grid_h, w.grid_w], "d_k": dk,
                   "d_v": dv, "io_dtype": w.dtype, "calls_per_step": len(w.directions),
                   "timing": "eager" if args.eager else "hip graph replay"},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def swiglu_main(args):
    """One step = one Spatial SwiGLU block over the workload's grid (inputs resident in HBM)."""
    import torch

    import gla_inputs
    import recurrent_vision_backbone_chunkwise_amd as gla

    if not os.path.exists(gla.LIB_PATH):
        from recurrent_vision_backbone_chunkwise_amd import build as hip_build
        hip_build.build()
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
    w = gla_inputs.swiglu_workload(args.swiglu_workload)
    cpu_in = gla_inputs.make_swiglu_inputs(w.B, w.grid_h, w.grid_w, w.C, w.F, w.dtype, seed=w.seed)
    ins = [t.to("cuda:0") for t in cpu_in]
    out = torch.empty_like(ins[0])
    stream = torch.cuda.Stream()

    def step():
        gla.gtr_swiglu_fwd(*ins, out, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        graph.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(args.steps):
            graph.replay() if graph is not None else step()
        stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    tokens = w.B * w.n_tok
    value = tokens / (ms_per_step * 1e-3)

    gla.gtr_gla_profile_begin()
    with torch.cuda.stream(stream):
        for _ in range(args.profile_steps):
            step()
    prof = gla.gtr_gla_profile_end()
    torch.cuda.synchronize()
    kern = {n: 1e3 * ms / c for n, (ms, c) in prof.items() if c > 0}
    elt = 4 if w.dtype == "f32" else 2
    M, C, F = tokens, w.C, w.F
    # algorithmic work per launch: GEMM flops; the mix kernel reads u once (fp16 for fp16 I/O,
    # else fp32) and writes h once
    work = {
        "swiglu_gemm_in": ("mfma", 2.0 * M * C * 2 * F),
        "swiglu_gemm_out": ("mfma", 2.0 * M * F * C),
        "swiglu_mix": ("hbm", float(M * (2 * F * (2 if w.dtype == "f16" else 4) + F * elt) + 10 * F * elt)),
    }
    per = {}
    for name, us in kern.items():
        bound, amount = work[name]
        if bound == "mfma":
            ach, peak, unit = amount / (us * 1e-6) / 1e12, MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
        else:
            ach, peak, unit = amount / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
        per[name] = {"avg_us": round(us, 3), "bound": bound, "achieved": round(ach, 1), "peak": peak,
                     "unit": unit, "frac": round(ach / peak, 4)}
    dominant = max(kern, key=kern.get)
    d = per[dominant]
    roofline = {"bound": d["bound"], "kernel": dominant, "achieved": d["achieved"], "peak": d["peak"],
                "unit": d["unit"], "frac": d["frac"], "traffic": None, "kernels": per}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import swiglu as oracle_swiglu
        rows = max(1, min(w.grid_h, int(args.cpu_seconds * 4)))
        sample = [cpu_in[0][:, :rows].contiguous()] + list(cpu_in[1:])
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle_swiglu.spatial_swiglu(*sample)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 1000:
                break
        t = time.perf_counter() - t0
        cpu = {"value": round(reps * w.B * rows * w.grid_w / t, 1), "unit": "tokens/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"the first {rows} grid rows of {w.name} x {reps} repetitions, {t:.1f} s, "
                         "fp64 numpy (BLAS threads as the host provides)"}
    line = {
        "metric": "Spatial SwiGLU block tokens/sec (B*N), one MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "grid": [w.grid_h, w.grid_w], "C": C, "F": F,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
