#!/usr/bin/env python3
"""Benchmark of the triangle multiplicative update on one MI355X.

One step = the outgoing update and the incoming update (each: input gate,
contraction, output gate) on one seeded synthetic batch resident in HBM.
Prints ONE JSON line:
  value         TFLOP/s over the step (matmul flops of both directions)
  roofline      the dominant kernel's algorithmic GB/s (or TFLOP/s) against the
                MI355X peak; its duration from HIP events recorded after every
                kernel in a second timed region of K steps
  cpu_baseline  the fp64 oracle timed on this host (rank 0, N=1 only)
With --chained the step is the pair update in model order instead (outgoing with
its residual add, then incoming on that result with its residual add); the
per-kernel region still times the plain stages.

The timed steps launch their six kernels one by one; --launch graph captures the
step once in a HIP graph and times replays of it instead (the eager step time is
reported in both cases). The per-kernel region always launches eagerly.

With --op attention the step is triangular attention around the starting node, then
around the ending node (each with its own weights, 4 heads of width 32) on the same
workload's z and mask; per-kernel events time its two kernels (projection, attention).
With --op transition the step is the pair transition instead (one kernel: LayerNorm,
c_z -> 2 c_z -> c_z with ReLU, masked residual) on the same workload's z and mask; its
line reports pair-updates/s with the same roofline and cpu_baseline objects.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--chained]
                    [--launch graph|eager] [--op trimul|transition] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "triangle-mult-update TFLOP/s & pair-updates/s at N=512,c_z=128 bf16 (1 GPU)"
TRANSITION_METRIC = "pair-transition pair-updates/s (expansion 2, masked residual, 1 GPU)"
ATTENTION_METRIC = "triangular-attention pair-updates/s (starting+ending node, 4 heads of 32, 1 GPU)"
KERNELS = ("k1_input_gate", "k2_contract", "k3_output_gate")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# A bounded spin on the GPU queued ahead of each per-kernel event region, so the host has
# enqueued the region's launches before the GPU reaches them: the event pair around a
# kernel then brackets the kernel, not the host's launch gap.
HOST_AHEAD_CYCLES = 20_000_000


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # the GPU's clocks settle only after some 100 ms of sustained work: 200 untimed steps
    # (about 60 ms of the headline step, more for attention) before the timed region
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default=None)
    p.add_argument("--chained", action="store_true",
                   help="time the pair update in model order instead: outgoing with its residual "
                        "add, then incoming on that result with its residual add")
    p.add_argument("--launch", choices=("eager", "graph"), default="eager",
                   help="timed steps launch their kernels one by one (default) or replay one "
                        "captured HIP graph of the step")
    p.add_argument("--op", choices=("trimul", "transition", "attention"), default="trimul",
                   help="time the triangle multiplicative update (default), the pair transition "
                        "or triangular attention")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-kernel-events", action="store_true",
                   help="time whole steps only (skip the per-kernel timed region)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run a plain device-to-device copy of this many MiB three times "
                        "(reference kernel for scaling HBM byte counters)")
    return p.parse_args()


def cpu_baseline(d, directions, threads, min_seconds=10.0, max_reps=8):
    """The fp64 oracle as it stands, on the same workload, both directions, repeated
    until about `min_seconds` of CPU time has passed. Returns (seconds per pass, passes)."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import tri_mul_ref
    z = torch.from_numpy(d["z"]).to(torch.bfloat16).to(torch.float64).numpy()
    reps, total = 0, 0.0
    with threadpool_limits(limits=threads):
        while reps < max_reps and (reps == 0 or total < min_seconds):
            t0 = time.perf_counter()
            for direction, w in directions:
                tri_mul_ref(z, d["mask"], w, direction)
            total += time.perf_counter() - t0
            reps += 1
    return total / reps, reps


def timed_steps(run, steps, stream):
    """Milliseconds per call of `run` over `steps` calls between two HIP events on
    `stream` (synchronised on both sides), and the wall seconds of the region."""
    import torch
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(steps):
        run()
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end) / steps, time.perf_counter() - wall0


def copy_calibration(mib, dev):
    """A plain device-to-device copy of `mib` MiB, three times (the reference kernel the
    HBM byte counters are scaled by); nothing when `mib` is 0."""
    if not mib:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def graph_of(step, dev):
    """`step` captured once in a HIP graph (after one run on a side stream)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph.replay()  # one untimed replay
    return graph


def roofline_of(kname, avg_ms, bytes_per_launch, flops_per_launch, dtype, traffic):
    from pair_rep_triangle_amd.metrics import MI355X_PEAK
    gbps = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    tfl = flops_per_launch / (avg_ms * 1e-3) / 1e12
    peak_fl = MI355X_PEAK["bf16_TFLOPs"] if dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
    ridge = peak_fl * 1e12 / (MI355X_PEAK["hbm_GBps"] * 1e9)
    if flops_per_launch / bytes_per_launch < ridge:
        return {"kernel": kname, "bound": "hbm", "achieved": round(gbps, 1),
                "peak": MI355X_PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": round(gbps / MI355X_PEAK["hbm_GBps"], 4), "traffic": traffic}
    return {"kernel": kname, "bound": "mfma", "achieved": round(tfl, 1), "peak": peak_fl,
            "unit": "TFLOP/s", "frac": round(tfl / peak_fl, 4), "traffic": traffic}


def bench_transition(args):
    """The pair transition (hidden = 2 c_z, the expansion the pages give for the pair
    track) on the workload's z and mask, out of place."""
    import numpy as np
    import torch
    from pair_rep_triangle_amd.inputs import HEADLINE, WORKLOADS, make_transition_weights, make_workload
    from pair_rep_triangle_amd.metrics import MI355X_PEAK, transition_work
    from pair_rep_triangle_amd.trimul import PairTransition

    name = args.workload or HEADLINE
    spec = WORKLOADS[name]
    d = make_workload(name, seed=args.seed)
    B, n, c_z, dtype = spec["batch"], spec["n"], spec["c_z"], spec["dtype"]
    hidden = 2 * c_z
    wt = make_transition_weights(np.random.default_rng(args.seed + 2), c_z, hidden, random_affine=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    z = torch.from_numpy(d["z"]).to(tdt).to(dev)
    mask = torch.from_numpy(d["mask"]).to(tdt).to(dev)
    mod = PairTransition(wt, c_z, hidden, dtype)
    out = torch.empty_like(z)
    stream = torch.cuda.current_stream(dev)

    def step():
        mod.forward(z, mask, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    copy_calibration(args.copy_calibration_mb, dev)
    ms_eager, wall = timed_steps(step, args.steps, stream)
    ms_step, launch = ms_eager, "eager"
    if args.launch == "graph":
        graph = graph_of(step, dev)
        ms_step, wall = timed_steps(graph.replay, args.steps, stream)
        launch = "hipgraph"

    # the kernel alone: a HIP event before and after each launch
    kernels, roofline = {}, None
    pairs = B * n * n
    wk = transition_work(c_z, hidden, esz)
    if not args.no_kernel_events:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda._sleep(HOST_AHEAD_CYCLES)
        for a, b in evs:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in evs])
        avg_ms = float(per.mean())
        bytes_l, flops_l = wk["bytes"] * pairs, wk["flops"] * pairs
        roofline = roofline_of("pair_transition", avg_ms, bytes_l, flops_l, dtype,
                               measured_traffic(name, "pair_transition"))
        peak_fl = MI355X_PEAK["bf16_TFLOPs"] if dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
        kernels["pair_transition"] = {
            "avg_us": round(avg_ms * 1e3, 3), "median_us": round(float(np.median(per)) * 1e3, 3),
            "GBps": round(bytes_l / (avg_ms * 1e-3) / 1e9, 1),
            "TFLOPs": round(flops_l / (avg_ms * 1e-3) / 1e12, 1),
            "hbm_frac": round(bytes_l / (avg_ms * 1e-3) / 1e9 / MI355X_PEAK["hbm_GBps"], 4),
            "mfma_frac": round(flops_l / (avg_ms * 1e-3) / 1e12 / peak_fl, 4),
            "bytes_per_launch": bytes_l, "flops_per_launch": flops_l,
        }

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import pair_transition_ref
        threads = min(16, len(os.sched_getaffinity(0)))
        zh = torch.from_numpy(d["z"]).to(torch.bfloat16).to(torch.float64).numpy()
        reps, total = 0, 0.0
        with threadpool_limits(limits=threads):
            while reps < 8 and (reps == 0 or total < 10.0):
                t0 = time.perf_counter()
                pair_transition_ref(zh, d["mask"], wt)
                total += time.perf_counter() - t0
                reps += 1
        dt = total / reps
        cpu = {"value": round(pairs / dt, 1), "unit": "pair-updates/s", "cores": threads,
               "kind": "oracle", "seconds_per_pass": round(dt, 3),
               "sample": f"whole workload {name}, fp64 NumPy oracle (BLAS on {threads} "
                         f"threads), {reps} passes averaged"}

    rec = {
        "metric": TRANSITION_METRIC, "value": round(pairs / (ms_step * 1e-3), 1),
        "unit": "pair-updates/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "ms_per_step_eager": round(ms_eager, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"pair_transition_{name}", "batch": B, "n": n, "c_z": c_z,
                   "hidden": hidden, "mask": spec["mask"], "launch": launch},
        "tflops": round(wk["flops"] * pairs / (ms_step * 1e-3) / 1e12, 2),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_attention(args):
    """Triangular attention around both nodes (4 heads of 32) on the workload's z and mask."""
    import numpy as np
    import torch
    from pair_rep_triangle_amd.inputs import HEADLINE, WORKLOADS, make_attention_weights, make_workload
    from pair_rep_triangle_amd.metrics import MI355X_EXP_PER_S, MI355X_PEAK, attention_work
    from pair_rep_triangle_amd.trimul import TriAttention

    name = args.workload or HEADLINE
    spec = WORKLOADS[name]
    d = make_workload(name, seed=args.seed)
    B, n, c_z, dtype = spec["batch"], spec["n"], spec["c_z"], spec["dtype"]
    heads, hdim = 4, 32
    if dtype != "bf16":
        print("bench.py: triangular attention runs in bf16 only", file=sys.stderr)
        sys.exit(2)
    ws_nodes = {node: make_attention_weights(np.random.default_rng(args.seed + 3 + i), c_z, heads,
                                             hdim, random_affine=True)
                for i, node in enumerate(("starting", "ending"))}
    dev = torch.device("cuda:0")
    z = torch.from_numpy(d["z"]).to(torch.bfloat16).to(dev)
    mask = torch.from_numpy(d["mask"]).to(torch.bfloat16).to(dev)
    mods = {node: TriAttention(w, c_z, heads, hdim) for node, w in ws_nodes.items()}
    ws = mods["starting"].new_workspace(B, n, dev)
    outs = {node: torch.empty_like(z) for node in mods}
    stream = torch.cuda.current_stream(dev)

    def step():
        for node, mod in mods.items():
            mod.forward(z, mask, out=outs[node], node=node, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    copy_calibration(args.copy_calibration_mb, dev)
    ms_eager, wall = timed_steps(step, args.steps, stream)
    ms_step, launch = ms_eager, "eager"
    if args.launch == "graph":
        graph = graph_of(step, dev)
        ms_step, wall = timed_steps(graph.replay, args.steps, stream)
        launch = "hipgraph"

    pairs = B * n * n
    work = attention_work(n, c_z, heads, hdim, 2)
    kernels, roofline = {}, None
    if not args.no_kernel_events:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda._sleep(HOST_AHEAD_CYCLES)
        for k in range(args.steps):
            evs[k][0].record(stream)
            e = 1
            for node, mod in mods.items():
                for st in (1, 2):
                    mod.stage(st, z, mask, out=outs[node], node=node, workspace=ws)
                    evs[k][e].record(stream)
                    e += 1
        torch.cuda.synchronize()
        per = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(4)]
                        for k in range(args.steps)])
        for idx, kname in enumerate(("ka_project", "ka_core")):
            samples = np.concatenate([per[:, idx], per[:, idx + 2]])  # both nodes
            avg_ms = float(samples.mean())
            wk = work[kname]
            gbps = wk["bytes"] * pairs / (avg_ms * 1e-3) / 1e9
            tfl = wk["flops"] * pairs / (avg_ms * 1e-3) / 1e12
            kd = {"avg_us": round(avg_ms * 1e3, 3), "median_us": round(float(np.median(samples)) * 1e3, 3),
                  "GBps": round(gbps, 1), "TFLOPs": round(tfl, 1),
                  "hbm_frac": round(gbps / MI355X_PEAK["hbm_GBps"], 4),
                  "mfma_frac": round(tfl / MI355X_PEAK["bf16_TFLOPs"], 4),
                  "bytes_per_launch": int(wk["bytes"] * pairs), "flops_per_launch": wk["flops"] * pairs}
            if "exps" in wk:
                ges = wk["exps"] * pairs / (avg_ms * 1e-3) / 1e9
                kd["Gexp_per_s"] = round(ges, 1)
                kd["exp_frac"] = round(ges * 1e9 / MI355X_EXP_PER_S, 4)
            kernels[kname] = kd
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        kd = kernels[dom]
        traffic = measured_traffic(name, dom)
        if dom == "ka_core":
            roofline = {"kernel": dom, "bound": "alu", "achieved": kd["Gexp_per_s"],
                        "peak": round(MI355X_EXP_PER_S / 1e9, 1), "unit": "Gexp/s",
                        "frac": kd["exp_frac"], "traffic": traffic}
        else:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": kd["GBps"],
                        "peak": MI355X_PEAK["hbm_GBps"], "unit": "GB/s",
                        "frac": kd["hbm_frac"], "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import tri_attention_ref
        threads = min(16, len(os.sched_getaffinity(0)))
        zh = torch.from_numpy(d["z"]).to(torch.bfloat16).to(torch.float64).numpy()
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            tri_attention_ref(zh, d["mask"], ws_nodes["starting"], "starting")
            dt = time.perf_counter() - t0
        cpu = {"value": round(pairs / dt, 1), "unit": "pair-updates/s", "cores": threads,
               "kind": "oracle", "seconds_per_pass": round(dt, 2),
               "sample": f"the starting node over the whole workload {name}, fp64 NumPy "
                         f"oracle (BLAS on {threads} threads), one pass"}

    flops_pair = work["ka_project"]["flops"] + work["ka_core"]["flops"]
    rec = {
        "metric": ATTENTION_METRIC, "value": round(2 * pairs / (ms_step * 1e-3), 1),
        "unit": "pair-updates/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"triangular_attention_{name}", "batch": B, "n": n, "c_z": c_z,
                   "heads": heads, "head_dim": hdim, "nodes": "starting+ending",
                   "mask": spec["mask"], "launch": launch},
        "tflops": round(2 * flops_pair * pairs / (ms_step * 1e-3) / 1e12, 2),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the operator is not sharded "
              "across GPUs (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.op == "transition":
        bench_transition(args)
        return
    if args.op == "attention":
        bench_attention(args)
        return

    import numpy as np
    import torch
    from pair_rep_triangle_amd.inputs import HEADLINE, WORKLOADS, make_weights, make_workload
    from pair_rep_triangle_amd.metrics import MI355X_PEAK, flops_per_pair, kernel_work
    from pair_rep_triangle_amd.trimul import TriMul

    name = args.workload or HEADLINE
    spec = WORKLOADS[name]
    d = make_workload(name, seed=args.seed)
    B, n, c_z, c, dtype = spec["batch"], spec["n"], spec["c_z"], spec["c"], spec["dtype"]
    w_out = d["weights"]
    w_in = make_weights(np.random.default_rng(args.seed + 1), c_z, c)  # second module
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    esz = 2 if dtype == "bf16" else 4

    dev = torch.device("cuda:0")
    z = torch.from_numpy(d["z"]).to(tdt).to(dev)
    mask = torch.from_numpy(d["mask"]).to(tdt).to(dev)
    mods = [("outgoing", TriMul(w_out, c_z, c, dtype)), ("incoming", TriMul(w_in, c_z, c, dtype))]
    ws = mods[0][1].new_workspace(B, n, device=dev)
    outs = [torch.empty_like(z) for _ in mods]
    stream = torch.cuda.current_stream(dev)

    def step():
        if args.chained:  # z -> outs[0] = z + upd_out(z) -> outs[1] = outs[0] + upd_in(outs[0])
            mods[0][1].forward_residual(z, mask, out=outs[0], direction="outgoing", workspace=ws)
            mods[1][1].forward_residual(outs[0], mask, out=outs[1], direction="incoming",
                                        workspace=ws)
            return
        for (direction, mod), out in zip(mods, outs):
            mod.forward(z, mask, out=out, direction=direction, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    copy_calibration(args.copy_calibration_mb, dev)

    # timed region 1: K whole steps (outgoing + incoming), HIP events on the launch stream;
    # eager launches, then (--launch graph) the same step captured once and replayed K times
    ms_eager, wall = timed_steps(step, args.steps, stream)
    ms_step, launch = ms_eager, "eager"
    if args.launch == "graph":
        graph = graph_of(step, dev)
        ms_step, wall = timed_steps(graph.replay, args.steps, stream)
        launch = "hipgraph"

    # timed region 2: the same K steps again with a HIP event after every kernel (on the
    # launch stream), for each kernel's duration inside the real K1 -> K2 -> K3 order.
    # Kept apart from region 1 because every event adds a marker packet to the stream.
    # The host queues it while the GPU runs a short spin, so no launch gap is timed.
    per_kernel_ms = {}
    if not args.no_kernel_events:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
        torch.cuda._sleep(HOST_AHEAD_CYCLES)
        for k in range(args.steps):
            evs[k][0].record(stream)
            e = 1
            for (direction, mod), out in zip(mods, outs):
                for s_idx in (1, 2, 3):
                    mod.stage(s_idx, z, mask, out=out, direction=direction, workspace=ws)
                    evs[k][e].record(stream)
                    e += 1
        torch.cuda.synchronize()
        per = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(6)]
                        for k in range(args.steps)])
        for idx, kname in enumerate(KERNELS):
            samples = np.concatenate([per[:, idx], per[:, idx + 3]])  # both directions
            per_kernel_ms[kname] = (float(samples.mean()), float(np.median(samples)))

    pairs = B * n * n
    fl_dir = flops_per_pair(n, c_z, c) * pairs
    tflops = 2 * fl_dir / (ms_step * 1e-3) / 1e12
    pair_updates = 2 * pairs / (ms_step * 1e-3)

    work = kernel_work(n, c_z, c, esz)
    kernels = {}
    for kname, (avg_ms, med_ms) in per_kernel_ms.items():
        wk = work[kname]
        gbps = wk["bytes"] * pairs / (avg_ms * 1e-3) / 1e9
        tfl = wk["flops"] * pairs / (avg_ms * 1e-3) / 1e12
        ai = wk["flops"] / wk["bytes"]
        peak_fl = MI355X_PEAK["bf16_TFLOPs"] if dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
        ridge = peak_fl * 1e12 / (MI355X_PEAK["hbm_GBps"] * 1e9)
        bound = "hbm" if ai < ridge else "mfma"
        kernels[kname] = {
            "avg_us": round(avg_ms * 1e3, 3), "median_us": round(med_ms * 1e3, 3), "GBps": round(gbps, 1), "TFLOPs": round(tfl, 1),
            "hbm_frac": round(gbps / MI355X_PEAK["hbm_GBps"], 4),
            "mfma_frac": round(tfl / peak_fl, 4), "bound": bound,
            "bytes_per_launch": wk["bytes"] * pairs, "flops_per_launch": wk["flops"] * pairs,
        }

    roofline = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        kd = kernels[dom]
        traffic = measured_traffic(name, dom)
        if kd["bound"] == "hbm":
            roofline = {"kernel": dom, "bound": "hbm", "achieved": kd["GBps"],
                        "peak": MI355X_PEAK["hbm_GBps"], "unit": "GB/s",
                        "frac": round(kd["GBps"] / MI355X_PEAK["hbm_GBps"], 4), "traffic": traffic}
        else:
            pk = MI355X_PEAK["bf16_TFLOPs"] if dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
            roofline = {"kernel": dom, "bound": "mfma", "achieved": kd["TFLOPs"], "peak": pk,
                        "unit": "TFLOP/s", "frac": round(kd["TFLOPs"] / pk, 4), "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        dt, reps = cpu_baseline(d, [("outgoing", w_out), ("incoming", w_in)], threads)
        cpu = {"value": round(2 * fl_dir / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "seconds_per_pass": round(dt, 2),
               "pair_updates_per_s": round(2 * pairs / dt, 1),
               "sample": f"whole workload {name}, outgoing + incoming, fp64 NumPy oracle "
                         f"(BLAS on {threads} threads), {reps} passes averaged"}

    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "n": n, "c_z": c_z, "c": c,
                   "valid_length": d["meta"].get("valid_length", n),
                   "directions": ("outgoing->incoming, chained with residual adds"
                                  if args.chained else "outgoing+incoming"),
                   "mask": spec["mask"], "launch": launch},
        "pair_updates_per_s": round(pair_updates, 1),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE table,
    or None when there is no row or the kernel source changed since it was taken."""
    from pair_rep_triangle_amd.profile_summary import source_sha
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                cells = [c.strip() for c in line.strip().strip("|").split("|")]
                if len(cells) == 6 and cells[0] == workload and cells[1] == kernel:
                    if cells[2] != source_sha(kernel):
                        return None
                    return int(float(cells[5]))
    except OSError:
        return None
    return None


if __name__ == "__main__":
    main()
