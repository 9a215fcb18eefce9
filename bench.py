#!/usr/bin/env python3
"""Benchmark of the split-K W4A16 group-128 matmul on one MI355X.

Workload (one "step"): the Qwen3-4B prefill projection sweep -- q 2560->4096,
k/v 2560->1024, o 4096->2560, gate/up 2560->9728, down 9728->2560, each at
M = 16, 32, 64, 128, 2048 rows -- 35 W4A16 g128 matmuls, each with the split
count the MI355X occupancy policy picks (split kernel + reduce, or the unsplit
kernel). Inputs are synthetic and seeded (A ~ N(0,1) bf16, q ~ U{0..15},
scale ~ U[0.005, 0.02] bf16, bias = -8*scale) and resident in HBM before
timing starts.

Timing:
  * the step is captured once as a HIP graph per rotation set and replayed
    (two sets, so consecutive replays read different buffers; one step touches
    ~0.5 GB, more than the 256 MB Infinity Cache, so each matmul reads cold);
    W warm-up steps, then K timed steps between two synchronisations;
  * per shape: a graph of R back-to-back calls over R distinct buffer sets
    totalling >= 1 GiB, for the policy's split and for the unsplit control;
  * the dominant kernel (largest share of the step) is also timed launch by
    launch with HIP events on its stream, for the roofline figure.

CPU baseline: the fp64 CPU oracle on the host cores, on a bounded sample of
the same sweep (listed in the output), extrapolated to one whole sweep.

Prints ONE JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split-K W4A16 matmul µs + % HBM/MFMA roofline, Qwen3-4B projections M=16–2048"
HBM_PEAK = 8.0e12          # bytes/s, MI355X published
MFMA_BF16_PEAK = 2.5e15    # flop/s, MI355X published dense bf16
ROTATE_BYTES = 1 << 30     # distinct bytes per per-shape rotation


def algorithmic_bytes(M, N, K):
    """Bytes any W4A16 g128 implementation must move: packed weights, scale+bias, A, C."""
    return N * K // 2 + N * (K // 128) * 4 + 2 * M * K + 2 * M * N


def algorithmic_flops(M, N, K):
    return 2 * M * N * K


def roofline(M, N, K, seconds):
    b, f = algorithmic_bytes(M, N, K), algorithmic_flops(M, N, K)
    t_hbm, t_mfma = b / HBM_PEAK, f / MFMA_BF16_PEAK
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return dict(bytes=b, flops=f, bound=bound, t_roof_us=max(t_hbm, t_mfma) * 1e6,
                frac=max(t_hbm, t_mfma) / seconds, gbs=b / seconds / 1e9, tflops=f / seconds / 1e12)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline sample budget")
    ap.add_argument("--no-per-shape", action="store_true")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    return ap.parse_args()


class Shape:
    """Device buffers of one projection shape: R input sets, one output, one workspace."""

    def __init__(self, name, M, N, K, idx, sets, torch, syn, q):
        self.name, self.M, self.N, self.K, self.idx = name, M, N, K, idx
        self.q = q
        self.plan = q.qmm_splitk_plan(M, N, K)
        self.s = self.plan.s
        d = syn.w4a16_weights(N, K, seed=2000 + idx)
        A = syn.normal_bf16((M, K), seed=2500 + idx)

        def dev16(x):
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()

        base = (dev16(A), torch.from_numpy(d["Wq"].view("int32")).cuda(), dev16(d["scale"]), dev16(d["bias"]))
        self.sets = [base] + [tuple(t.clone() for t in base) for _ in range(sets - 1)]
        self.C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty(max(q.w4a16_workspace_bytes(M, N, self.s), 256), dtype=torch.uint8, device="cuda")

    def call(self, r, s):
        A, W, S, B = self.sets[r % len(self.sets)]
        self.q.qmm_w4a16_g128(A, W, S, B, self.C, self.M, self.N, self.K, s,
                              self.ws if s > 1 else None, self.ws.numel() if s > 1 else 0)

    def set_bytes(self):
        return algorithmic_bytes(self.M, self.N, self.K)

    def free(self):
        self.sets = []


def graph_of(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the caches of everything the capture will touch
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps=3):
    """Median seconds of one replay."""
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def per_shape(torch, syn, q, name, M, N, K, idx):
    """Per-call seconds of the policy split and of the unsplit control over >= 1 GiB of rotation."""
    probe = Shape(name, M, N, K, idx, 1, torch, syn, q)
    R = max(8, min(1024, math.ceil(ROTATE_BYTES / probe.set_bytes())))
    probe.free()
    sh = Shape(name, M, N, K, idx, R, torch, syn, q)
    out = {}
    for s in sorted({sh.s, 1}):
        g = graph_of(torch, lambda: [sh.call(r, s) for r in range(R)])
        out[s] = time_graph(torch, g) / R
        del g
    sh.free()
    torch.cuda.empty_cache()
    return sh, R, out


def cpu_baseline(syn, budget_s):
    """fp64 oracle on the host cores over a bounded, listed sample of the sweep, extrapolated."""
    import numpy as np
    import oracle

    cores = oracle.default_threads()
    shapes = syn.projection_sweep()
    # order: small-M shapes whole, then 128-row slices of the 2048-row shapes
    order = [sh for sh in shapes if sh[1] <= 128] + [sh for sh in shapes if sh[1] > 128]
    spent, sample, est_total = 0.0, [], 0.0
    done_macs, done_time = 0.0, 0.0
    for name, M, N, K, idx in order:
        rows = M if M <= 128 else 128
        if spent >= budget_s:
            break
        d = syn.w4a16_weights(N, K, seed=2000 + idx)
        A = syn.normal_bf16((rows, K), seed=2500 + idx)
        t0 = time.perf_counter()
        oracle.qmm_w4a16(A, d["Wq"], d["scale"], d["bias"], rows, N, K, s=1, nthreads=cores)
        dt = time.perf_counter() - t0
        spent += dt
        sample.append("%s M=%d%s" % (name, M, "" if rows == M else " (rows 0..%d)" % (rows - 1)))
        est_total += dt * (M / rows)
        done_macs += rows * N * K
        done_time += dt
    covered = {(s.split()[0], s.split()[1]) for s in sample}
    rate = done_time / done_macs  # seconds per MAC over the sample
    for name, M, N, K, idx in shapes:
        if (name, "M=%d" % M) not in covered:
            est_total += rate * M * N * K
    return dict(value=est_total * 1e6, unit="us per sweep (35 projection matmuls, extrapolated)", cores=cores,
                kind="oracle",
                sample="%s; %.1f s measured, rest extrapolated by multiply-add count" % (", ".join(sample), spent))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch

    import qmm_synth as syn
    import weight_only_quantized_qmm_amd as q

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    q.lib()
    sweep = syn.projection_sweep()

    # ---- the timed step: the whole sweep, graph-replayed over two rotation sets
    shapes = [Shape(n, M, N, K, i, 2, torch, syn, q) for n, M, N, K, i in sweep]
    graphs = [graph_of(torch, lambda r=r: [sh.call(r, sh.s) for sh in shapes]) for r in range(2)]
    for i in range(args.warmup):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        graphs[i % 2].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = e0.elapsed_time(e1) / 1e3 / args.steps

    # eager step (host launch overhead included), for reference
    for sh in shapes:
        sh.call(0, sh.s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(3):
        for sh in shapes:
            sh.call(i, sh.s)
    torch.cuda.synchronize()
    eager_step_s = (time.perf_counter() - t0) / 3

    # ---- the dominant kernel: the unsplit large-M launches, timed one by one with events
    dom = [sh for sh in shapes if sh.M > 128 and sh.s == 1]
    durs, flops, nbytes = [], [], []
    stream = torch.cuda.current_stream()
    for rep in range(3):
        for sh in dom:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sh.call(rep + 1, 1)
            b.record(stream)
            b.synchronize()
            if rep > 0:  # first pass warms
                durs.append(a.elapsed_time(b) / 1e3)
                flops.append(algorithmic_flops(sh.M, sh.N, sh.K))
                nbytes.append(algorithmic_bytes(sh.M, sh.N, sh.K))
    del graphs
    for sh in shapes:
        sh.free()
    torch.cuda.empty_cache()
    avg_dur = sum(durs) / len(durs)
    achieved = sum(flops) / len(flops) / avg_dur
    roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK, "traffic": None,
            "kernel": "w4a16 kernel, unsplit, M=2048 launches (%s)" % ", ".join(sh.name for sh in dom),
            "launches": len(durs), "avg_launch_us": avg_dur * 1e6,
            "block_tile": [dom[0].plan.block_m, dom[0].plan.block_n] if dom else None}

    # ---- per-shape table
    table = []
    if not args.no_per_shape:
        for n, M, N, K, i in sweep:
            sh, R, t = per_shape(torch, syn, q, n, M, N, K, i)
            r = roofline(M, N, K, t[sh.s])
            table.append(dict(name=n, M=M, N=N, K=K, s=sh.s, us=round(t[sh.s] * 1e6, 3),
                              us_unsplit=round(t[1] * 1e6, 3), speedup_vs_unsplit=round(t[1] / t[sh.s], 3),
                              tflops=round(r["tflops"], 2), gbs=round(r["gbs"], 1), bound=r["bound"],
                              roof_us=round(r["t_roof_us"], 3), frac=round(r["frac"], 4), rotation_sets=R))
            print("# %s" % json.dumps(table[-1]), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(syn, args.cpu_seconds)

    pol = q.policy_preset("QMM_POLICY_MI355X").as_dict()
    line = {
        "metric": METRIC,
        "value": round(step_s * 1e6, 3),
        "unit": "us per sweep (35 W4A16 g128 projection matmuls, split + reduce included)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-4B projection sweep: q,k,v,o,gate,up,down x M in {16,32,64,128,2048}, "
                               "W4A16 g128, MI355X policy split",
                   "shapes": len(sweep), "policy": pol, "timing": "hipGraph replay of the whole sweep",
                   "wall_s_timed": round(wall, 4)},
        "eager_us_per_step": round(eager_step_s * 1e6, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
        "shapes": table,
    }
    if table:
        small = [t for t in table if t["M"] <= 128]
        line["summary"] = {
            "small_M_mean_frac": round(sum(t["frac"] for t in small) / len(small), 4),
            "M2048_mean_frac": round(sum(t["frac"] for t in table if t["M"] == 2048) / 7, 4),
            "split_never_slower": all(t["speedup_vs_unsplit"] >= 0.98 for t in table),
            "sum_per_shape_us": round(sum(t["us"] for t in table), 2),
        }
    text = json.dumps(line)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
