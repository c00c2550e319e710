"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--act-quant mxfp8]

A step is one moe_forward (router + top-k, dispatch, grouped expert FFN up
and down, combine) over one batch of synthetic tokens already resident in
HBM.  W untimed steps (by default at least 10 and a quarter second of them,
so that a short layer is not timed while the clock ramps up under load),
then K timed steps between device synchronisations;
the expert weights rotate over several identical copies so that each step
reads them from HBM rather than from the 256 MB last-level cache.

Printed (one JSON line on stdout): tokens/s of the layer, plus
  roofline     -- the dominant kernel (the grouped up-projection with the
                  SwiGLU epilogue, 2/3 of the FLOPs) timed with HIP events
                  on its stream over K launches, against the bf16 dense MFMA
                  peak (decode workloads: against HBM bandwidth); traffic is
                  the HBM bytes per launch from the committed rocprofv3
                  counter summary under profiles/,
  cpu_baseline -- the float64 CPU oracle on a bounded token sample of the
                  same workload, on this host's cores.
With --act-quant mxfp8 (MXFP4 workloads) the layer runs in the W4A8 mode:
the experts' input and hidden are MXFP8 and both projections run on the
scaled MFMA; the prefill roofline is then against the dense FP8 peak (the
FP8 x FP4 MFMA issues at the FP8 rate), and the oracle runs the same mode.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % HBM peak (decode) / % MFMA peak (prefill)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(L, counts, act_quant=None):
    """FLOPs of the routed layer and HBM bytes of what it must read/write."""
    n, d, E, k, f = L["n"], L["d"], L["E"], L["k"], L["d_ff"]
    R = n * k
    flops_up = 4.0 * R * d * f
    flops = 2.0 * n * d * E + flops_up + 2.0 * R * f * d
    act_b = 2 if L["x_dtype"] == "bf16" else 4
    if L["w_dtype"] == "mxfp4":
        per_expert = 3 * d * f // 2 + 3 * d * f // 32
    else:
        per_expert = 3 * d * f * (2 if L["w_dtype"] == "bf16" else 4)
    active = int((counts > 0).sum())
    bytes_ = E * d * act_b + 2 * n * d * act_b + active * per_expert
    if act_quant:  # MXFP8 rows in and out: a byte per value plus a scale per 32
        up_bytes = active * (2 * d * f * (per_expert / (3 * d * f))) + (n * d + R * f) * 33 / 32
    else:
        up_bytes = active * (2 * d * f * (per_expert / (3 * d * f))) + n * d * act_b + R * f * 2
    return {"flops": flops, "flops_up": flops_up, "bytes": bytes_, "up_bytes": up_bytes,
            "active_experts": active}


def cpu_baseline(L, budget_s=15.0, threads=16, act_quant=None):
    """Time the float64 oracle on a token sample: a probe on 64 tokens sizes
    the sample to about budget_s seconds; a sample that is the whole batch is
    repeated until about 10 s of work have been timed."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    with threadpool_limits(limits=threads):
        m = min(L["n"], 64)
        t0 = time.perf_counter()
        oracle.forward(L, L["k"], L["renorm"], rows=np.arange(m), act_quant=act_quant)
        dt = time.perf_counter() - t0
        if dt < budget_s / 3 and m < L["n"]:
            m = int(min(L["n"], max(m, m * budget_s / max(dt, 1e-3))))
        runs, total = 0, 0.0
        while runs == 0 or total < 10.0:
            t0 = time.perf_counter()
            oracle.forward(L, L["k"], L["renorm"], rows=np.arange(m), act_quant=act_quant)
            total += time.perf_counter() - t0
            runs += 1
        info = threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] + [1])
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info
                             if i.get("user_api") == "blas"})) or "unknown BLAS"
    return {"value": m * runs / total, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"float64 dense-then-masked oracle on the first {m} of {L['n']} tokens "
                      f"(all {L['E']} experts per token{', W4A8 mode' if act_quant else ''}), "
                      f"{runs} run(s), {total:.2f} s; host {cpu_model()} "
                      f"({os.cpu_count()} logical CPUs), numpy {np.__version__} on {blas}"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before timing (default: at least 10 and 0.25 s of them, "
                         "so that the clock has settled under load)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--act-quant", choices=["mxfp8"], default=None,
                    help="W4A8 mode of an MXFP4 layer (MXFP8 expert inputs and hidden)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one HIP graph that holds one step per weight copy "
                         "(consecutive layers with distinct weights) instead of eager launches")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit; "
                         "run under rocprofv3 --pmc to scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {nbytes} bytes 3 times")
        return

    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd import workloads as W
    from mixture_experts_layer_wave_amd.profiling import read_traffic
    from mixture_experts_layer_wave_amd.device import DeviceLayer, to_device

    # Default: the largest single-GPU layer, the Mixtral-shaped top-2 prefill.
    name = args.workload or W.MIXTRAL
    wl = W.WORKLOADS[name]
    log(f"[bench] workload {name}: generating inputs")
    L = W.make_layer(name, cache=False)
    torch.cuda.set_device(0)
    aq = args.act_quant
    if aq and wl.wdt != "mxfp4":
        print("--act-quant needs an MXFP4 workload", file=sys.stderr)
        sys.exit(2)
    D = DeviceLayer(L, act_quant=aq)
    stream = torch.cuda.current_stream()

    # Identical weight copies in distinct HBM buffers, rotated per step.
    copies = [D.weights]
    keep = []
    for _ in range(max(0, args.copies - 1)):
        ws = {key: (None if D.w[key] is None else D.w[key].clone()) for key in D.w}
        keep.append(ws)
        copies.append(B.ExpertWeights(D.weights.dtype, *(B._ptr(ws[key]) for key in ("w1", "w3", "w2", "s1", "s3", "s2")),
                                      None, 0, D.weights.act_quant))

    def step(i, st=stream):
        B.moe_forward(D.shape, D.x, D.act, D.wg, D.bias, copies[i % len(copies)], D.y, D.act,
                      D.idx, D.topw, D.ws, D.ws_bytes, st)

    if args.warmup is not None:
        warm = args.warmup
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
    else:
        # Steps in groups of ten until a quarter second has run: a short layer
        # would otherwise be timed while the clock still ramps up under load.
        warm = 0
        w0 = time.perf_counter()
        while warm < 10 or time.perf_counter() - w0 < 0.25:
            for _ in range(10):
                step(warm)
                warm += 1
            torch.cuda.synchronize()
    per_launch = 1
    if args.graph:
        # One graph holds len(copies) consecutive steps, each on its own weight
        # copy; it is captured on a side stream and replayed on the launch stream.
        per_launch = len(copies)
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            for i in range(per_launch):
                step(i, cap)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for i in range(per_launch):
                    step(i, cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        for _ in range(max(1, warm // per_launch)):
            graph.replay()
        torch.cuda.synchronize()
    launches = max(1, args.steps // per_launch)
    steps_timed = launches * per_launch

    def launch(i):
        if args.graph:
            graph.replay()
        else:
            step(i)

    # The timed steps run back to back between two events on the launch
    # stream (an event between steps costs a few microseconds, a tenth of a
    # small decode step).
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(launches):
        launch(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / steps_timed
    # The per-step spread (p10/p50/p90) comes from a second pass with an
    # event at every launch boundary (so it includes their cost).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    marks[0].record(stream)
    for i in range(launches):
        launch(i)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(launches)]) / per_launch
    pct = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    log(f"[bench] {steps_timed} steps{' in graph replays' if args.graph else ''}: {ms_per_step * 1e3:.1f} us/step (wall {wall / steps_timed * 1e6:.1f} us/step)")

    # Routing of this batch (for the work model and the dominant-kernel loop).
    n, E, k = D.n, D.E, D.k
    R = n * k
    logits = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((n, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(R, dtype=torch.int32, device="cuda")
    inv = torch.empty((n, k), dtype=torch.int32, device="cuda")
    B.moe_router_topk(D.shape, D.x, D.act, D.wg, D.bias, logits, idx, tw, stream)
    B.moe_dispatch(D.shape, idx, counts, offsets, perm, inv, None, D.act, None, None, 0, stream)
    a_in, a_dt = D.x, D.act
    if aq:  # the up projection of the mode takes the MXFP8 tokens, writes an MXFP8 hidden
        a_in = torch.empty(B.moe_mxfp8_bytes(n, D.d), dtype=torch.uint8, device="cuda")
        B.moe_quantize_mxfp8(n, D.d, D.x, D.act, a_in, stream)
        a_dt = aq
        h = torch.empty(B.moe_mxfp8_bytes(R, D.d_ff), dtype=torch.uint8, device="cuda")
    else:
        h = torch.empty((R, D.d_ff), dtype=torch.int16 if D.wdt != "f32" else torch.float32, device="cuda")
    torch.cuda.synchronize()
    work = algorithmic_work(L, counts.cpu().numpy(), aq)
    decode = wl.wdt == "mxfp4" and wl.n <= 64

    # Dominant kernel: the grouped up-projection, one launch per call.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(min(warm, 2 * args.steps)):
        B.moe_expert_up(D.shape, a_in, a_dt, perm, offsets, copies[i % len(copies)], h, stream)
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        B.moe_expert_up(D.shape, a_in, a_dt, perm, offsets, copies[i % len(copies)], h, stream)
        b.record(stream)
    torch.cuda.synchronize()
    up_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    if decode:
        achieved = work["up_bytes"] / (up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = work["flops_up"] / (up_ms * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if aq else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch of this kernel from the committed rocprofv3
    # FETCH_SIZE / WRITE_SIZE summary (null once the kernel's sources change).
    if decode:
        fam = "mx_decode_kernel"
    elif wl.wdt == "mxfp4" and aq:
        fam = "mxw_gemm_kernel"  # W4A8 prefill: MXFP4 codes in LDS, MXFP8 activations
    elif wl.wdt == "mxfp4":
        fam = "mxw16_pair_kernel"  # W4A16 prefill up: 64- and 128-row tiles, two workgroups per CU
    else:
        fam = "big_gemm_kernel"
    traffic, src = read_traffic(name, fam, aq)
    roof["traffic"] = traffic
    roof["traffic_source"] = src
    roof["kernel"] = f"{fam}<up> (moe_expert_up)"
    roof["kernel_us"] = up_ms * 1e3
    log(f"[bench] up kernel {up_ms * 1e3:.1f} us -> {roof['achieved']:.1f} {roof['unit']} ({100 * roof['frac']:.1f}% of peak)")
    layer_tflops = work["flops"] / (ms_per_step * 1e-3) / 1e12
    layer_gbs = work["bytes"] / (ms_per_step * 1e-3) / 1e9
    # The whole step against the same roofline: algorithmic flops (prefill) or
    # bytes (decode) of the layer per step time.
    layer_frac = (layer_gbs / PEAK_HBM_GBS if decode else
                  layer_tflops / (PEAK_FP8_TFLOPS if aq else PEAK_BF16_TFLOPS))
    roof["layer_frac"] = layer_frac
    log(f"[bench] whole layer {layer_tflops:.1f} TFLOP/s, {layer_gbs:.1f} GB/s algorithmic "
        f"({100 * layer_frac:.1f}% of peak); active experts {work['active_experts']}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        cpu = cpu_baseline(L, act_quant=aq)
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    value = n / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps_timed, "warmup": warm, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": (D.act if D.wdt != "mxfp4" else
                  "mxfp8 x mxfp4 (w4a8)" if aq else "bf16 (mxfp4 weights)"),
        "data": "synthetic",
        "config": {"workload": name, "n": wl.n, "d": wl.d, "E": wl.E, "k": wl.k, "d_ff": wl.d_ff,
                   "weights": wl.wdt, "activations": wl.act, "act_quant": aq,
                   "weight_copies": len(copies), "hip_graph": bool(args.graph),
                   "layer_tflops": layer_tflops},
        "step_ms": pct,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)

    # Release the device state before the interpreter exits: the queued work,
    # the graph and every device buffer go now, while the HIP runtime (and a
    # profiler attached to it) is still fully up.
    torch.cuda.synchronize()
    if args.graph:
        del graph
    del copies, keep, D, evs, marks
    del logits, idx, tw, counts, offsets, perm, inv, h, a_in
    import gc

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
