#!/usr/bin/env python3
"""Benchmark of the triangle multiplicative update on one MI355X.

One step = the outgoing update and the incoming update (each: input gate,
contraction, output gate) on one seeded synthetic batch resident in HBM.
In order, the run
  1. measures peaks on this GPU (a 1 GiB device-to-device copy, a vendor bf16 GEMM);
  2. times every other workload once in its own launch configuration (the
     `workloads` table: step time, p10/median/p90, TFLOP/s, fraction of the
     3-kernel floor, per-kernel fractions of HBM and MFMA peak), which keeps the
     GPU busy so that the headline runs at the clocks of sustained work;
  3. times the headline workload: W untimed warm-up steps, then exactly K steps
     between two HIP events -> ms_per_step and value;
  4. times each kernel of the headline alone (K back-to-back launches of its stage
     between two HIP events, per direction), each kernel in the real K1 -> K2 -> K3
     order (a HIP event after every kernel), and each step with its own HIP events;
  5. times the fp64 oracle on this host.
Prints ONE JSON line:
  value         TFLOP/s over the step (matmul flops of both directions)
  roofline      the dominant kernel's algorithmic GB/s (or TFLOP/s) against the
                MI355X peak (and against the measured peak); its duration from the
                back-to-back launches of step 4 (an event between two kernels adds the
                marker's own gap to each; the in-order figures are `kernels_in_order`)
  cpu_baseline  the fp64 oracle timed on this host (rank 0, N=1 only)
With --chained the step is the pair update in model order instead (outgoing with
its residual add, then incoming on that result with its residual add); the
per-kernel region still times the plain stages.

The timed steps launch their six kernels one by one; --launch graph captures the
step once in a HIP graph and times replays of it instead (the eager step time is
reported in both cases). The per-kernel region always launches eagerly.

With --op attention the step is triangular attention around the starting node, then
around the ending node (each with its own weights, 4 heads of width 32) on the same
workload's z and mask; back-to-back launches of each stage time its two kernels
(projection, attention).
With --op transition the step is the pair transition instead (one kernel: LayerNorm,
c_z -> 2 c_z -> c_z with ReLU, masked residual) on the same workload's z and mask; its
line reports pair-updates/s with the same roofline and cpu_baseline objects.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--chained]
                    [--launch graph|eager] [--op trimul|transition|attention]
                    [--no-cpu-baseline] [--no-kernel-events] [--no-table]
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
    p.add_argument("--no-table", action="store_true",
                   help="skip the measured peaks and the other workloads' table")
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

    # the kernel alone: the step is one launch, so the eager timed region (K back-to-back
    # launches between two HIP events) is the kernel's own duration; per-launch events give
    # the median
    kernels, roofline = {}, None
    pairs = B * n * n
    wk = transition_work(c_z, hidden, esz)
    if not args.no_kernel_events:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in evs])
        avg_ms = ms_eager
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
        threads, affinity = cpu_threads()
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
               "affinity_cores": affinity,
               "sample": f"whole workload {name}, fp64 NumPy oracle (BLAS on {threads} "
                         f"threads: {cpu_thread_note(threads, affinity)}), {reps} passes averaged"}

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
        # each kernel alone: K back-to-back launches of its stage between two HIP events,
        # the stages in order per node (the projection leaves what the attention reads)
        regions = []
        for node, mod in mods.items():
            for st in (1, 2):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.steps):
                    mod.stage(st, z, mask, out=outs[node], node=node, workspace=ws)
                b.record(stream)
                regions.append((st - 1, a, b))
        torch.cuda.synchronize()
        per = {0: [], 1: []}
        for idx, a, b in regions:
            per[idx].append(a.elapsed_time(b) / args.steps)
        for idx, kname in enumerate(("ka_project", "ka_core")):
            samples = np.array(per[idx])  # one average per node
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
        threads, affinity = cpu_threads()
        zh = torch.from_numpy(d["z"]).to(torch.bfloat16).to(torch.float64).numpy()
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            tri_attention_ref(zh, d["mask"], ws_nodes["starting"], "starting")
            dt = time.perf_counter() - t0
        cpu = {"value": round(pairs / dt, 1), "unit": "pair-updates/s", "cores": threads,
               "kind": "oracle", "seconds_per_pass": round(dt, 2),
               "affinity_cores": affinity,
               "sample": f"the starting node over the whole workload {name}, fp64 NumPy "
                         f"oracle (BLAS on {threads} threads: "
                         f"{cpu_thread_note(threads, affinity)}), one pass"}

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


def measure_peaks(dev):
    """Peaks measured on this GPU beside the published ones: HBM bandwidth of a plain
    1 GiB device-to-device copy (read + write bytes over the event time, best of 5), and
    the vendor bf16 GEMM (torch.matmul, 8192^3, best of 5) as the reachable MFMA rate."""
    import torch
    stream = torch.cuda.current_stream(dev)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    copy_ms, gemm_ms = [], []
    for _ in range(5):
        for fn, acc in ((lambda: dst.copy_(src), copy_ms), (lambda: torch.matmul(a, b), gemm_ms)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            acc.append(e0.elapsed_time(e1))
    del src, dst, a, b
    return {"hbm_copy_GBps": round(2 * (1 << 30) / (min(copy_ms) * 1e-3) / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2 * 8192 ** 3 / (min(gemm_ms) * 1e-3) / 1e12, 1),
            "how": "1 GiB device-to-device copy (read + write bytes) and torch.matmul "
                   "8192x8192x8192 bf16, best of 5 each, HIP events"}


class TriMulBench:
    """One workload's modules, buffers and step for the multiplicative update."""

    def __init__(self, name, seed, dev, chained=False, skip=False):
        import numpy as np
        import torch
        from pair_rep_triangle_amd.inputs import WORKLOADS, make_weights, make_workload
        from pair_rep_triangle_amd.trimul import TriMul

        self.name, self.spec = name, WORKLOADS[name]
        self.d = make_workload(name, seed=seed)
        s = self.spec
        self.B, self.n, self.c_z, self.c, self.dtype = s["batch"], s["n"], s["c_z"], s["c"], s["dtype"]
        self.esz = 2 if self.dtype == "bf16" else 4
        self.w_out = self.d["weights"]
        self.w_in = make_weights(np.random.default_rng(seed + 1), self.c_z, self.c)  # 2nd module
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        self.z = torch.from_numpy(self.d["z"]).to(tdt).to(dev)
        self.mask = torch.from_numpy(self.d["mask"]).to(tdt).to(dev)
        self.mods = [("outgoing", TriMul(self.w_out, self.c_z, self.c, self.dtype)),
                     ("incoming", TriMul(self.w_in, self.c_z, self.c, self.dtype))]
        self.ws = self.mods[0][1].new_workspace(self.B, self.n, device=dev)
        self.outs = [torch.empty_like(self.z) for _ in self.mods]
        self.stream = torch.cuda.current_stream(dev)
        self.chained = chained
        # with skip, a step first computes the mask extents (once, for both updates) and
        # both updates skip the contraction past each item's extent
        self.skip = skip
        self.extents = torch.empty((self.B, 64), dtype=torch.int32, device=dev)

    def step(self):
        from pair_rep_triangle_amd.trimul import mask_extents
        mods, outs, z, mask, ws = self.mods, self.outs, self.z, self.mask, self.ws
        ext = mask_extents(mask, out=self.extents) if self.skip else None
        if self.chained:  # z -> outs[0] = z + upd_out(z) -> outs[1] = outs[0] + upd_in(outs[0])
            mods[0][1].forward_residual(z, mask, out=outs[0], direction="outgoing", workspace=ws,
                                        extents=ext)
            mods[1][1].forward_residual(outs[0], mask, out=outs[1], direction="incoming",
                                        workspace=ws, extents=ext)
            return
        for (direction, mod), out in zip(mods, outs):
            mod.forward(z, mask, out=out, direction=direction, workspace=ws, extents=ext)

    def valid_lengths(self):
        meta = self.d["meta"]
        if "valid_lengths" in meta:
            return list(meta["valid_lengths"])
        return [meta.get("valid_length", self.n)] * self.B

    def useful_flops_per_step(self):
        """Matmul flops of both directions counted over each item's valid L x L pairs
        with the contraction over its L residues (the work that remains when padding is
        skipped)."""
        from pair_rep_triangle_amd.metrics import flops_per_pair
        return 2 * sum(L * L * flops_per_pair(L, self.c_z, self.c) for L in self.valid_lengths())

    @property
    def pairs(self):
        return self.B * self.n * self.n

    def flops_per_step(self):
        from pair_rep_triangle_amd.metrics import flops_per_pair
        return 2 * flops_per_pair(self.n, self.c_z, self.c) * self.pairs

    def floor_ms(self):
        """The 3-kernel floor of one step: per kernel the larger of its algorithmic bytes
        over the HBM peak and its flops over the MFMA peak, both directions."""
        from pair_rep_triangle_amd.metrics import MI355X_PEAK, kernel_work
        peak = MI355X_PEAK["bf16_TFLOPs"] if self.dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
        t = 0.0
        for wk in kernel_work(self.n, self.c_z, self.c, self.esz).values():
            t += max(wk["bytes"] * self.pairs / (MI355X_PEAK["hbm_GBps"] * 1e9),
                     wk["flops"] * self.pairs / (peak * 1e12))
        return 2 * t * 1e3

    def kernel_times_isolated(self, reps):
        """Each kernel alone: `reps` back-to-back launches of its stage between two HIP
        events on the launch stream, the stages in order per direction (K1 leaves the
        operands K2 reads, K2 the product K3 reads), all regions enqueued before one
        synchronisation so the GPU stays busy. No event sits between two launches of a
        region. {kernel: the per-direction average durations in ms}."""
        import numpy as np
        import torch
        regions = []
        for (direction, mod), out in zip(self.mods, self.outs):
            for s_idx, kname in zip((1, 2, 3), KERNELS):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(self.stream)
                for _ in range(reps):
                    mod.stage(s_idx, self.z, self.mask, out=out, direction=direction,
                              workspace=self.ws)
                b.record(self.stream)
                regions.append((kname, a, b))
        torch.cuda.synchronize()
        res = {k: [] for k in KERNELS}
        for kname, a, b in regions:
            res[kname].append(a.elapsed_time(b) / reps)
        return {k: np.array(v) for k, v in res.items()}

    def kernel_times(self, steps):
        """Each kernel's duration in the real K1 -> K2 -> K3 order: a HIP event after every
        kernel on the launch stream. The host enqueues a step (six launches, seven events)
        in a small fraction of the step's GPU time, so after the first step the queue runs
        ahead of the GPU and no launch gap is timed. {kernel: samples in ms over both
        directions}."""
        import numpy as np
        import torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for k in range(steps):
            evs[k][0].record(self.stream)
            e = 1
            for (direction, mod), out in zip(self.mods, self.outs):
                for s_idx in (1, 2, 3):
                    mod.stage(s_idx, self.z, self.mask, out=out, direction=direction,
                              workspace=self.ws)
                    evs[k][e].record(self.stream)
                    e += 1
        torch.cuda.synchronize()
        per = np.array([[evs[k][j].elapsed_time(evs[k][j + 1]) for j in range(6)]
                        for k in range(steps)])
        return {kname: np.concatenate([per[:, i], per[:, i + 3]]) for i, kname in enumerate(KERNELS)}

    def step_times(self, steps):
        """Each whole step between its own pair of HIP events."""
        import numpy as np
        import torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record(self.stream)
            self.step()
            b.record(self.stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    def kernel_report(self, samples):
        from pair_rep_triangle_amd.metrics import MI355X_PEAK, kernel_work
        import numpy as np
        work = kernel_work(self.n, self.c_z, self.c, self.esz)
        peak_fl = MI355X_PEAK["bf16_TFLOPs"] if self.dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
        ridge = peak_fl * 1e12 / (MI355X_PEAK["hbm_GBps"] * 1e9)
        kernels = {}
        for kname, smp in samples.items():
            avg_ms, med_ms = float(smp.mean()), float(np.median(smp))
            wk = work[kname]
            gbps = wk["bytes"] * self.pairs / (avg_ms * 1e-3) / 1e9
            tfl = wk["flops"] * self.pairs / (avg_ms * 1e-3) / 1e12
            kernels[kname] = {
                "avg_us": round(avg_ms * 1e3, 3), "median_us": round(med_ms * 1e3, 3),
                "GBps": round(gbps, 1), "TFLOPs": round(tfl, 1),
                "hbm_frac": round(gbps / MI355X_PEAK["hbm_GBps"], 4),
                "mfma_frac": round(tfl / peak_fl, 4),
                "bound": "hbm" if wk["flops"] / wk["bytes"] < ridge else "mfma",
                "bytes_per_launch": wk["bytes"] * self.pairs,
                "flops_per_launch": wk["flops"] * self.pairs,
            }
        return kernels

    def summary(self, ms_step, step_samples, kernels):
        import numpy as np
        self.last_ms = ms_step
        fl = self.flops_per_step()
        rec = {"ms_per_step": round(ms_step, 4),
               "TFLOPs": round(fl / (ms_step * 1e-3) / 1e12, 2),
               "pair_updates_per_s": round(2 * self.pairs / (ms_step * 1e-3), 1),
               "floor_ms": round(self.floor_ms(), 4),
               "floor_frac": round(self.floor_ms() / ms_step, 4)}
        if step_samples is not None:
            rec["step_ms_p10_median_p90"] = [round(float(np.percentile(step_samples, q)), 4)
                                             for q in (10, 50, 90)]
        if kernels:
            rec["kernels"] = {k: {f: v[f] for f in ("avg_us", "hbm_frac", "mfma_frac", "bound")}
                              for k, v in kernels.items()}
        return rec

    def close(self):
        for _, mod in self.mods:
            mod.close()


def skip_summary(wb, args):
    """The same workload's step with mask-extent skipping: the extents computed once per
    step, both updates skipping past each item's extent."""
    wb.skip = True
    for _ in range(max(args.warmup, 3)):
        wb.step()
    ms, _ = timed_steps(wb.step, args.steps, wb.stream)
    wb.skip = False
    useful = wb.useful_flops_per_step()
    return {"skip": {"ms_per_step": round(ms, 4),
                     "speedup": round(wb.last_ms / ms, 3) if getattr(wb, "last_ms", None) else None,
                     "useful_TFLOPs": round(useful / (ms * 1e-3) / 1e12, 2),
                     "valid_lengths": wb.valid_lengths()}}


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

    import torch
    from pair_rep_triangle_amd.inputs import HEADLINE, WORKLOADS
    from pair_rep_triangle_amd.metrics import MI355X_PEAK

    name = args.workload or HEADLINE
    dev = torch.device("cuda:0")
    # the headline's inputs go to the GPU first: building them on the host takes a while,
    # and the GPU's clocks drop while it idles, so its timed steps must follow GPU work
    hb = TriMulBench(name, args.seed, dev, chained=args.chained)

    # 1. peaks measured on this GPU
    peaks = measure_peaks(dev) if not args.no_table else None

    # 2. every other workload once, each in the launch configuration of its own bench line
    #    (K steps after max(W, 3) warm-up steps, then per-kernel and per-step events). The
    #    GPU is busy throughout, so the headline below runs at the clocks of sustained work.
    table = {}
    if not args.no_table:
        for other in WORKLOADS:
            if other == name:
                continue
            wb = TriMulBench(other, args.seed, dev)
            for _ in range(max(args.warmup, 3)):
                wb.step()
            ms, _ = timed_steps(wb.step, args.steps, wb.stream)
            table[other] = wb.summary(ms, wb.step_times(args.steps),
                                      wb.kernel_report(wb.kernel_times_isolated(args.steps)))
            if wb.spec["mask"] in ("block", "lengths"):
                table[other].update(skip_summary(wb, args))
            wb.close()
            del wb
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    # 3. the headline: W untimed warm-up steps, then exactly K timed steps
    for _ in range(args.warmup):
        hb.step()
    torch.cuda.synchronize()
    copy_calibration(args.copy_calibration_mb, dev)
    ms_eager, wall = timed_steps(hb.step, args.steps, hb.stream)
    ms_step, launch = ms_eager, "eager"
    if args.launch == "graph":
        graph = graph_of(hb.step, dev)
        ms_step, wall = timed_steps(graph.replay, args.steps, hb.stream)
        launch = "hipgraph"

    # 4. per-kernel and per-step event regions of the same workload (kept apart from the
    #    timed region: every event adds a marker packet to the stream)
    kernels, kernels_in_order, step_samples = {}, {}, None
    if not args.no_kernel_events:
        kernels = hb.kernel_report(hb.kernel_times_isolated(args.steps))
        kernels_in_order = {k: {f: v[f] for f in ("avg_us", "median_us", "hbm_frac", "mfma_frac")}
                            for k, v in hb.kernel_report(hb.kernel_times(args.steps)).items()}
        step_samples = hb.step_times(args.steps)

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
            pk = MI355X_PEAK["bf16_TFLOPs"] if hb.dtype == "bf16" else MI355X_PEAK["fp32_mfma_TFLOPs"]
            roofline = {"kernel": dom, "bound": "mfma", "achieved": kd["TFLOPs"], "peak": pk,
                        "unit": "TFLOP/s", "frac": round(kd["TFLOPs"] / pk, 4), "traffic": traffic}
        if peaks:
            roofline["frac_of_measured_peak"] = round(
                kd["GBps"] / peaks["hbm_copy_GBps"] if kd["bound"] == "hbm"
                else kd["TFLOPs"] / peaks["bf16_gemm_TFLOPs"], 4)

    # 5. the oracle on the host
    cpu = None
    if not args.no_cpu_baseline:
        threads, affinity = cpu_threads()
        dt, reps = cpu_baseline(hb.d, [("outgoing", hb.w_out), ("incoming", hb.w_in)], threads)
        fl = hb.flops_per_step()
        cpu = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "seconds_per_pass": round(dt, 2),
               "pair_updates_per_s": round(2 * hb.pairs / dt, 1), "affinity_cores": affinity,
               "sample": f"whole workload {name}, outgoing + incoming, fp64 NumPy oracle "
                         f"(BLAS on {threads} threads: {cpu_thread_note(threads, affinity)}), "
                         f"{reps} passes averaged"}

    head = hb.summary(ms_step, step_samples, kernels)
    table[name] = dict(head, headline=True)
    if not args.no_table and hb.spec["mask"] in ("block", "lengths") and not args.chained:
        table[name].update(skip_summary(hb, args))
    rec = {
        "metric": METRIC, "value": head["TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": hb.dtype,
        "data": "synthetic",
        "config": {"workload": name, "batch": hb.B, "n": hb.n, "c_z": hb.c_z, "c": hb.c,
                   "valid_length": hb.d["meta"].get("valid_length", hb.n),
                   "directions": ("outgoing->incoming, chained with residual adds"
                                  if args.chained else "outgoing+incoming"),
                   "mask": hb.spec["mask"], "launch": launch},
        "pair_updates_per_s": head["pair_updates_per_s"],
        "floor_frac": head["floor_frac"],
        "step_ms_p10_median_p90": head.get("step_ms_p10_median_p90"),
        "wall_s": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "kernels_in_order": kernels_in_order,
        "measured_peaks": peaks,
        "workloads": table,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_threads():
    """Threads for the oracle: every core in the process's affinity, capped by the host's
    CPU share when the environment sets one (OMP_NUM_THREADS). Returns (threads, affinity)."""
    affinity = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(share)) if share and share.isdigit() and int(share) > 0 else affinity
    return threads, affinity


def cpu_thread_note(threads, affinity):
    if threads == affinity:
        return "every core in the affinity mask"
    return f"the host's CPU share OMP_NUM_THREADS={threads} of {affinity} cores in the affinity mask"


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE table,
    or None when there is no row or the kernel source changed since it was taken. A
    kernel with a second form (the streamed output gate, the wide transition) has its
    own row under that form's name; a workload runs one form, so the first row found
    for the workload among the kernel's names is the one."""
    from pair_rep_triangle_amd.profile_summary import source_sha
    names = {"k3_output_gate": ("k3_output_gate_stream", "k3_output_gate"),
             "pair_transition": ("pair_transition_wide", "pair_transition")}.get(kernel, (kernel,))
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for name in names:
        for line in lines:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) == 6 and cells[0] == workload and cells[1] == name:
                if cells[2] != source_sha(name):
                    return None
                return int(float(cells[5]))
    return None


if __name__ == "__main__":
    main()
