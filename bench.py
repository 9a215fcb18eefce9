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
  * the dominant kernel (largest share of the step: the large-M kernel) is
    timed on its own for the roofline figure: its first-pass launches of the
    seven M = 2048 shapes with the plan's decomposition, back to back in one
    graph, HIP events on the launch stream around each replay
    (``--dominant-only`` runs just this part, for the profiler);
  * machine floors measured in the same run (libqmm_calib.so): empty-kernel
    dispatch, HBM stream read and copy, bf16 MFMA rate, and the large-M kernel's
    step loop without global memory; for every M <= 128 shape, a plain read of
    its bytes and that read followed by a dependent store (its practical floors).

Counters: ``--pmc-run [large|small]`` is the workload of rocprofv3 --pmc passes.
For the dominant kernel, two passes (FETCH_SIZE, WRITE_SIZE) turn into the text
summary under profiles/ that the ``traffic`` field reads back (``--summarize-pmc``;
it stays null when the kernel source changed after the counters were taken), and
two more (MIX_COUNTERS) into its instruction mix and unit utilisation
(``--summarize-mix``); one pass of LDS counters over ``--dominant-only`` sets its
LDS activity beside that of the step-loop calibration (``--summarize-lds``). For
the small-M kernel, FETCH_SIZE and WRITE_SIZE passes and a kernel trace give its
per-launch HBM traffic and rate (``--summarize-small-pmc``).

CPU baseline: the fp64 CPU oracle on the host cores, on a bounded sample of
the same sweep (listed in the output), extrapolated to one whole sweep, plus the
oracle on one thread for the 32 x 1024 x 2560 K-projection case.

Output: the last line on stdout is ONE compact JSON line (the headline: metric,
value, dominant-kernel roofline, CPU baseline, summary of the per-shape table).
The tables (per shape, dense sweep, decode, formats, decode attention, stream-K)
go to the JSON file named by --tables-out; stderr carries short progress lines.
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


def algorithmic_bytes(M, N, K, bits=4, group=128):
    """Bytes any implementation of the weight-only format must move: packed codes,
    scale+bias, A, C (W4A16 g128 by default)."""
    return N * K * bits // 8 + N * (K // group) * 4 + 2 * M * K + 2 * M * N


def algorithmic_flops(M, N, K):
    return 2 * M * N * K


def roofline(M, N, K, seconds, bits=4, group=128):
    b, f = algorithmic_bytes(M, N, K, bits, group), algorithmic_flops(M, N, K)
    t_hbm, t_mfma = b / HBM_PEAK, f / MFMA_BF16_PEAK
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return dict(bytes=b, flops=f, bound=bound, t_roof_us=max(t_hbm, t_mfma) * 1e6,
                frac=max(t_hbm, t_mfma) / seconds, gbs=b / seconds / 1e9, tflops=f / seconds / 1e12)


# The dominant kernel of the step (largest share of its time): the large-M W4A16 kernel.
DOMINANT_KERNEL = "w4a16_wide_kernel"
# What the committed traffic counters were taken on: the kernel's source, the host code
# that plans its launches, and the workload of the counter passes.
DOMINANT_SOURCES = [os.path.join(ROOT, "weight_only_quantized_qmm_amd", "csrc", f)
                    for f in ("qmm_w4a16_wide.hip", "qmm_api.cpp", "qmm_launch.h", "qmm_device.h")]
DOMINANT_WORKLOAD = "first pass (qmm_w4a16_g128_pass1) of the plan, M=2048 q,k,v,o,gate,up,down"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "w4a16_wide_M2048_traffic.txt")
STEP_LOOP_STEPS = 2048     # steps per workgroup of the step-loop calibration
COPY_BYTES = 256 << 20     # size of the plain copy that calibrates the profiler's byte counters


def progress(kind, row, keys):
    """One short progress line on stderr (plain text, never JSON)."""
    print("# %s %s" % (kind, " ".join("%s=%s" % (k, row[k]) for k in keys if k in row)), file=sys.stderr, flush=True)


def dominant_shapes(shapes):
    """The M = 2048 shapes: the large-M kernel runs them."""
    return [sh for sh in shapes if sh.M > 128]


def source_digest(paths=None):
    """Digest of the dominant kernel's sources (code only: comments and whitespace are
    dropped, so an edited comment leaves it unchanged) and of the counter workload."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in (paths or DOMINANT_SOURCES):
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    h.update(DOMINANT_WORKLOAD.encode())
    return h.hexdigest()[:16]


def calib_lib():
    import ctypes
    path = os.path.join(ROOT, "weight_only_quantized_qmm_amd", "libqmm_calib.so")
    if not os.path.exists(path):
        raise RuntimeError("libqmm_calib.so is not built; run python -m weight_only_quantized_qmm_amd.build")
    L = ctypes.CDLL(path)
    I, P, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.qmm_calib_empty.argtypes = [I, P]
    L.qmm_calib_read.argtypes = [P, S, P, P]
    L.qmm_calib_read_grid.argtypes = [P, S, I, P, P]
    L.qmm_calib_chain.argtypes = [P, S, I, P, P]
    L.qmm_calib_copy.argtypes = [P, P, S, P]
    L.qmm_calib_mfma.argtypes = [I, I, P, P]
    L.qmm_calib_step.argtypes = [I, I, I, I, I, P, P]
    for f in (L.qmm_calib_empty, L.qmm_calib_read, L.qmm_calib_read_grid, L.qmm_calib_chain, L.qmm_calib_copy,
              L.qmm_calib_mfma, L.qmm_calib_step):
        f.restype = I
    return L


def calibrate(torch):
    """This GPU's own floors, measured in the same run: dispatch, HBM read/copy, bf16 MFMA."""
    L = calib_lib()
    out = torch.zeros(4, dtype=torch.int32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        g = graph_of(torch, lambda: [fn() for _ in range(reps)])
        return time_graph(torch, g) / reps

    t_empty = timed(lambda: L.qmm_calib_empty(1, torch.cuda.current_stream().cuda_stream), 200)
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf2 = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    t_read = timed(lambda: L.qmm_calib_read(buf.data_ptr(), nbytes, out.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream), 4)
    t_copy = timed(lambda: L.qmm_calib_copy(buf.data_ptr(), buf2.data_ptr(), nbytes // 2,
                                            torch.cuda.current_stream().cuda_stream), 4)
    del buf, buf2
    grid, iters = 256 * 8, 4096
    t_mfma = timed(lambda: L.qmm_calib_mfma(grid, iters, out.data_ptr(), torch.cuda.current_stream().cuda_stream), 4)
    step_grid, steps = 256, STEP_LOOP_STEPS
    step = {}
    for layout, lname in ((0, "w256x32"), (1, "w128x64")):
        step[lname] = {}
        for name, lds_reads, dequant in (("mfma", 0, 0), ("mfma_lds", 1, 0), ("mfma_dequant", 0, 1),
                                         ("mfma_lds_dequant", 1, 1)):
            t = timed(lambda: L.qmm_calib_step(step_grid, steps, layout, lds_reads, dequant, out.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream), 4)
            step[lname][name] = round(step_grid * 8 * steps * 8 * 32768 / t / 1e12, 1)
    torch.cuda.empty_cache()
    return {"empty_dispatch_us": round(t_empty * 1e6, 3),
            "hbm_read_TBps": round(nbytes / t_read / 1e12, 3),
            "hbm_copy_TBps": round(nbytes / t_copy / 1e12, 3),  # bytes read + bytes written
            "mfma_bf16_tflops": round(grid * 4 * iters * 4 * 32768 / t_mfma / 1e12, 1),
            "step_loop_tflops": step,
            "note": "empty kernel back to back in a graph; 2 GiB read; 1 GiB copy; "
                    "v_mfma_f32_32x32x16_bf16 loop on 2048 workgroups; step loop: the large-M kernel's "
                    "step (8 waves per CU, 8 MFMAs per wave and step) without global memory, in its "
                    "256 x 32 waves (8 LDS operand reads, 1 dequantised word) and in 128 x 64 waves "
                    "(4 reads, 2 words), with neither, either or both"}


def stream_floors(torch, sizes):
    """Practical floors of the HBM-bound calls, seconds per call for `nbytes`: a plain
    streaming read (libqmm_calib's read kernel on max(1024, nbytes/4096) workgroups, 16 bytes
    per load) and the same read followed by a dependent one-dword store per thread (the
    load -> store chain every matmul call has), each call on its own slice of a 1 GiB pool,
    as the per-shape timings rotate their inputs so that no call finds its bytes in a
    cache; {nbytes: (read seconds, chain seconds)}."""
    L = calib_lib()
    out = torch.zeros(8192 * 256, dtype=torch.int32, device="cuda")
    pool = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device="cuda")
    base = pool.data_ptr()
    res = {}
    for nbytes in sorted(set(sizes)):
        n = -(-nbytes // 256) * 256  # slices on 256-byte boundaries
        R = max(2, min(1024, ROTATE_BYTES // n))
        grid = min(8192, max(1024, -(-n // 4096)))
        t = []
        for fn in (L.qmm_calib_read_grid, L.qmm_calib_chain):
            g = graph_of(torch, lambda fn=fn: [fn(base + r * n, n, grid, out.data_ptr(),
                                                  torch.cuda.current_stream().cuda_stream) for r in range(R)])
            t.append(time_graph(torch, g) / R)
            del g
        res[nbytes] = tuple(t)
    del pool
    torch.cuda.empty_cache()
    return res


def read_traffic(alg_bytes_per_launch):
    """HBM bytes per launch of the dominant kernel from the committed profiler counters, or None.

    The summary records the digest of the kernel source it was taken on; a
    different digest (the kernel changed since) gives None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None, "no counter summary"
    fields = {}
    for line in open(TRAFFIC_SUMMARY):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel source digest") != source_digest():
        return None, "kernel, its launch plan or the counter workload changed since the counters were taken"
    t = float(fields["hbm bytes per launch (scaled)"])
    return t, "FETCH_SIZE + WRITE_SIZE per launch x copy-kernel scale; %.2fx the algorithmic bytes" % (
        t / alg_bytes_per_launch)


def dominant_roofline(torch, shapes, rounds=4):
    """Roofline figure of the dominant kernel: the large-M kernel's launch of every M = 2048
    shape exactly as the timed sweep makes it (the plan's decomposition), without the second
    pass: qmm_w4a16_g128_pass1, one kernel per call, `rounds` times over two buffer sets,
    captured as one graph; HIP events on the launch stream around each replay give the mean
    launch duration (median of the replays)."""
    dom = dominant_shapes(shapes)
    g = graph_of(torch, lambda: [sh.call_pass1(r) for r in range(rounds) for sh in dom])
    avg_dur = time_graph(torch, g) / (rounds * len(dom))
    del g
    flops = sum(algorithmic_flops(sh.M, sh.N, sh.K) for sh in dom) / len(dom)
    nbytes = sum(algorithmic_bytes(sh.M, sh.N, sh.K) for sh in dom) / len(dom)
    achieved = flops / avg_dur
    calib = calibrate(torch)
    traffic, traffic_note = read_traffic(nbytes)
    roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK, "traffic": traffic,
            "kernel": "%s as the plan launches it (first pass), M=2048 launches (%s)" % (
                DOMINANT_KERNEL, ", ".join("%s s=%d" % (sh.name, sh.s) for sh in dom)),
            "launches_per_replay": rounds * len(dom), "avg_launch_us": avg_dur * 1e6,
            "algorithmic_bytes_per_launch": nbytes, "flops_per_launch": flops,
            "frac_of_measured_mfma_peak": achieved / (calib["mfma_bf16_tflops"] * 1e12),
            "frac_of_step_loop": achieved / (calib["step_loop_tflops"]["w256x32"]["mfma_lds_dequant"] * 1e12),
            "traffic_note": traffic_note,
            "block_tiles": {sh.name: [sh.plan.block_m, sh.plan.block_n] for sh in dom}}
    return roof, calib


def dense_sweep(torch, syn, q):
    """Dense bf16 split-K, A, B bf16 [512, 16384]: us per call for each s of the sweep and
    for the library's own choice (s = 0), over >= 1 GiB of rotated inputs."""
    M = N = 512
    K = 16384
    d = syn.dense_inputs(M, N, K, seed=3000)

    def dev16(x):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    base = (dev16(d["A"]), dev16(d["B"]))
    R = max(8, math.ceil(ROTATE_BYTES / (2 * (M + N) * K)))
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(4 * 32 * M * N, dtype=torch.uint8, device="cuda")
    out = {}
    for s in (1, 2, 4, 6, 8, 12, 16, 32, 0):
        def run(s=s):
            for r in range(R):
                A, B = sets[r]
                q.qmm_bf16_splitk(A, B, C, M, N, K, s, ws if s != 1 else None, ws.numel() if s != 1 else 0)
        g = graph_of(torch, run)
        out["policy" if s == 0 else "s%d" % s] = round(time_graph(torch, g) / R * 1e6, 3)
        del g
    del sets, ws
    torch.cuda.empty_cache()
    byts, flops = 2 * (M + N) * K + 2 * M * N, 2 * M * N * K
    t = out["policy"] * 1e-6
    return {"shape": [M, N, K], "us": out, "roof_us": round(max(byts / HBM_PEAK, flops / MFMA_BF16_PEAK) * 1e6, 3),
            "frac_policy": round(max(byts / HBM_PEAK, flops / MFMA_BF16_PEAK) / t, 4)}


def decode_table(torch, syn, q):
    """Decode shapes (down, gate at M = 1, 4, 8): the matmul's policy split against its
    unsplit control and against the decode matrix-vector kernel (qmm_w4a16_gemv, its own
    split), with the weight-read rate (packed weights + scale/bias bytes / time)."""
    rows = []
    for name, M, N, K, idx in syn.decode_sweep():
        sh, R, t = per_shape(torch, syn, q, name, M, N, K, idx + 100)
        wbytes = N * K // 2 + N * (K // 128) * 4
        # the matrix-vector kernel over the same rotation
        gs = q.qmm_gemv_min_split(M, K)
        sh2 = Shape(name, M, N, K, idx + 100, R, torch, syn, q)
        ws = torch.empty(max(2 * gs * M * N, 256), dtype=torch.uint8, device="cuda")

        def run():
            for r in range(R):
                A, W, S, B = sh2.sets[r]
                q.qmm_w4a16_gemv(A, W, S, B, sh2.C, M, N, K, gs, ws if gs > 1 else None)
        g = graph_of(torch, run)
        t_gemv = time_graph(torch, g) / R
        del g
        sh2.free()
        torch.cuda.empty_cache()
        best = min(t[0], t_gemv)
        rows.append(dict(name=name, M=M, N=N, K=K, s=sh.s, us=round(t[0] * 1e6, 3), us_unsplit=round(t[1] * 1e6, 3),
                         gemv_s=gs, gemv_us=round(t_gemv * 1e6, 3),
                         weight_gbs=round(wbytes / best / 1e9, 1), weight_frac_hbm=round(wbytes / best / HBM_PEAK, 4)))
    return rows


def streamk_table(torch, syn, q, table):
    """The stream-K decomposition (qmm_w4a16_g128_streamk, default workgroups) on the
    M = 128 and 2048 sweep shapes, against the plan's time from the per-shape table."""
    plan_us = {(t["name"], t["M"]): t["us"] for t in table}
    rows = []
    for name, M, N, K, idx in syn.projection_sweep():
        if M < 128:
            continue
        probe = Shape(name, M, N, K, idx, 1, torch, syn, q)
        R = max(8, min(1024, math.ceil(ROTATE_BYTES / probe.set_bytes())))
        probe.free()
        sh = Shape(name, M, N, K, idx, R, torch, syn, q)
        nb = q.qmm_streamk_workspace_bytes(M, N, K, 0)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

        def run():
            for r in range(R):
                A, W, S, B = sh.sets[r]
                q.qmm_w4a16_g128_streamk(A, W, S, B, sh.C, M, N, K, 0, ws, nb)
        g = graph_of(torch, run)
        t = time_graph(torch, g) / R
        del g, ws
        sh.free()
        torch.cuda.empty_cache()
        r = roofline(M, N, K, t)
        rows.append(dict(name=name, M=M, us=round(t * 1e6, 3), plan_us=plan_us.get((name, M)),
                         workspace_mb=round(nb / 1e6, 1), frac=round(r["frac"], 4)))
        progress("streamk", rows[-1], ("name", "M", "us", "plan_us"))
    return rows


ATTN_SHAPES = [(1, 4096, 1), (1, 16384, 1), (8, 4096, 1), (32, 4096, 1), (32, 16384, 1), (8, 4096, 4)]


def attention_table(torch, q):
    """Split-KV decode attention on Qwen3-4B's heads (32 query heads, 8 key/value heads,
    head dimension 128) for (batch, cached keys, queries per request): µs per call under
    the library's split and unsplit, over >= 1 GiB of rotated caches, with the HBM
    roofline fraction of the algorithmic bytes (key and value rows read once, Q, O)."""
    Hq, Hkv, D = 32, 8, 128
    rows = []
    for B, L, Mq in ATTN_SHAPES:
        kv = 2 * B * Hkv * L * D * 2
        R = max(1, min(256, math.ceil(ROTATE_BYTES / kv)))
        gen = torch.Generator(device="cuda").manual_seed(4000 + B + L + Mq)
        sets = [tuple(torch.randn(*shape, device="cuda", generator=gen).to(torch.bfloat16)
                      for shape in ((B, Mq, Hq, D), (B, Hkv, L, D), (B, Hkv, L, D))) for _ in range(R)]
        lengths = torch.full((B,), L, dtype=torch.int32, device="cuda")
        O = torch.empty(B, Mq, Hq, D, dtype=torch.bfloat16, device="cuda")
        s_plan = q.qmm_attn_decode_split(B, Hkv, L)
        ws = torch.empty(max(q.qmm_attn_decode_workspace_bytes(B, Mq, Hq, s_plan), 16), dtype=torch.uint8,
                         device="cuda")
        t = {}
        for s in (0, 1):
            def run(s=s):
                for r in range(R):
                    Q, K, V = sets[r]
                    q.qmm_attn_decode(Q, K, V, lengths, O, B, Mq, Hq, Hkv, L, D, D ** -0.5, s,
                                      ws if (s or s_plan) > 1 else None)
            g = graph_of(torch, run)
            t[s] = time_graph(torch, g) / R
            del g
        del sets, ws
        torch.cuda.empty_cache()
        byts = kv + 2 * 2 * B * Mq * Hq * D
        rows.append(dict(B=B, L=L, Mq=Mq, Hq=Hq, Hkv=Hkv, D=D, s=s_plan, us=round(t[0] * 1e6, 3),
                         us_unsplit=round(t[1] * 1e6, 3), tbs=round(byts / t[0] / 1e12, 3),
                         frac_hbm=round(byts / HBM_PEAK / t[0], 4)))
        progress("attn", rows[-1], ("B", "L", "Mq", "s", "us", "frac_hbm"))
    return rows


FORMAT_VARIANTS = [((4, 128), True), ((4, 64), False), ((4, 32), False), ((8, 128), False), ((8, 64), False),
                   ((8, 32), False)]


def formats_table(torch, syn, q):
    """The other weight formats (qmm_wna16) and the fp32-partial option on the gate and
    down projections at M = 16, 128, 2048: µs per call under the library plan over >= 1 GiB
    of rotation, with the roofline fraction of the format's own algorithmic bytes."""
    rows = []
    for (bits, group), f32p in FORMAT_VARIANTS:
        for name, M, N, K, idx in syn.projection_sweep():
            if name not in ("gate", "down") or M not in (16, 128, 2048):
                continue
            sh, R, t = per_shape(torch, syn, q, name, M, N, K, idx + 500, fmt=(bits, group), f32p=f32p,
                                 unsplit=False)
            r = roofline(M, N, K, t[0], bits, group)
            rows.append(dict(bits=bits, group=group, partials="fp32" if f32p else "bf16", name=name, M=M, N=N, K=K,
                             s=sh.s, full_tiles=sh.plan.full_tiles, us=round(t[0] * 1e6, 3), bound=r["bound"],
                             gbs=round(r["gbs"], 1), tflops=round(r["tflops"], 2), frac=round(r["frac"], 4)))
            progress("format", rows[-1], ("bits", "group", "partials", "name", "M", "s", "us", "frac"))
    return rows


SMALL_KERNEL = "w4a16_skinny_kernel"
GEMV_KERNEL = "gemv_kernel"
DECODE_WORKLOAD = ("each decode shape (down, gate at M = 1, 4, 8) through the plan and through the matrix-vector "
                   "entry point, second of two rounds")
SMALL_WORKLOAD = ("the plan's call (matmul kernel, and the merge when split) of every sweep shape the small-M "
                  "kernel runs, second of two rounds")


def small_shapes():
    """The sweep shapes the small-M kernel runs (M <= 64, and q, k, v, o at M = 128)."""
    import weight_only_quantized_qmm_amd as q
    import qmm_synth as syn
    return [(n, M, N, K, i) for n, M, N, K, i in syn.projection_sweep() if q.qmm_splitk_plan(M, N, K).block_m < 128]


def pmc_run(kind="large"):
    """Workload of the counter passes. large: the first pass of each M = 2048 shape's plan
    once; small: the plan's whole call of each shape the small-M kernel runs, once. Then one
    plain copy (calibrates the byte counters)."""
    import torch
    import qmm_synth as syn
    import weight_only_quantized_qmm_amd as q
    torch.cuda.set_device(0)
    if kind == "large":
        shapes = [Shape(n, M, N, K, i, 1, torch, syn, q) for n, M, N, K, i in syn.projection_sweep() if M > 128]
        for sh in shapes:
            sh.call_pass1(0)
        what = "%d launches of %s" % (len(shapes), DOMINANT_KERNEL)
    elif kind == "decode":
        # two rounds over two buffer sets (the summary takes the second): each decode shape
        # through the plan (the small-M kernel, unsplit) and through the matrix-vector kernel
        shapes = [Shape(n, M, N, K, i + 100, 2, torch, syn, q) for n, M, N, K, i in syn.decode_sweep()]
        for r in range(2):
            for sh in shapes:
                sh.call(r, 0)
                torch.cuda.synchronize()
                gs = q.qmm_gemv_min_split(sh.M, sh.K)
                A, W, S, B = sh.sets[r]
                ws = torch.empty(max(2 * gs * sh.M * sh.N, 256), dtype=torch.uint8, device="cuda")
                q.qmm_w4a16_gemv(A, W, S, B, sh.C, sh.M, sh.N, sh.K, gs, ws if gs > 1 else None)
                torch.cuda.synchronize()
        what = "two rounds of %d decode shapes on %s and %s" % (len(shapes), SMALL_KERNEL, GEMV_KERNEL)
    else:
        # two rounds over two buffer sets: the second reads cold buffers with the clock up;
        # the summary takes its launches
        shapes = [Shape(n, M, N, K, i, 2, torch, syn, q) for n, M, N, K, i in small_shapes()]
        for r in range(2):
            for sh in shapes:
                sh.call(r, 0)
                torch.cuda.synchronize()
        what = "two rounds of %d calls on %s" % (len(shapes), SMALL_KERNEL)
    torch.cuda.synchronize()
    L = calib_lib()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    L.qmm_calib_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    print("pmc run: %s + one %d-byte copy" % (what, COPY_BYTES), flush=True)


def _counter_rows(d, counters):
    """{counter: [(dispatch id, kernel name, value)]} from a rocprofv3 --pmc output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    out = {c: [] for c in counters}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] in out:
                out[r["Counter_Name"]].append((int(r.get("Dispatch_Id") or 0), r["Kernel_Name"],
                                               float(r["Counter_Value"])))
    return {c: sorted(v) for c, v in out.items()}


def _trace_durations(d):
    """[(dispatch id, kernel name, ns)] from a rocprofv3 --kernel-trace output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % d)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return sorted(rows)


def summarize_small_pmc(fetch_dir, write_dir, trace_dir, commands):
    """Text summary of the small-M kernel's HBM traffic: FETCH_SIZE and WRITE_SIZE per launch
    (scaled by the copy kernel), beside the algorithmic bytes and, with the launch's duration
    from a kernel trace of the same workload, the achieved HBM rate."""
    fetch = _counter_rows(fetch_dir, ["FETCH_SIZE"])["FETCH_SIZE"]
    write = _counter_rows(write_dir, ["WRITE_SIZE"])["WRITE_SIZE"]
    trace = _trace_durations(trace_dir)
    pick = lambda rows, key: [v for _, k, v in rows if key in k]
    cf, cw = pick(fetch, "calib_copy"), pick(write, "calib_copy")
    f_scale, w_scale = COPY_BYTES / (cf[0] * 1024.0), COPY_BYTES / (cw[0] * 1024.0)
    import weight_only_quantized_qmm_amd as q
    shapes = small_shapes()
    # the second of the workload's two rounds
    df, dw, dt = [pick(rows, SMALL_KERNEL)[len(shapes):] for rows in (fetch, write, trace)]
    lines = ["# HBM traffic of %s (%s) from rocprofv3 counters" % (SMALL_KERNEL, SMALL_WORKLOAD),
             "commands:"] + ["  " + c for c in commands] + [
        "copy kernel: %d bytes read and written; FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB" % (COPY_BYTES, cf[0], cw[0]),
        "fetch scale: %.4f" % f_scale, "write scale: %.4f" % w_scale,
        "per launch of the matmul kernel (the merge kernel of split calls not included); bytes = scaled FETCH + WRITE;",
        "algorithmic = packed weights + scale/bias + A + C; us = kernel-trace duration of the same launch",
        "%-5s %5s %5s %5s %3s  %10s %10s %10s %6s %8s %8s" % ("proj", "M", "N", "K", "s", "fetch B", "write B",
                                                          "algo B", "ratio", "us", "HBM GB/s")]
    tot_b = tot_a = tot_t = 0.0
    for (n, M, N, K, _), fv, wv, ns in zip(shapes, df, dw, dt):
        s = q.qmm_splitk_plan(M, N, K).s
        fb, wb = fv * 1024 * f_scale, wv * 1024 * w_scale
        a = algorithmic_bytes(M, N, K)
        lines.append("%-5s %5d %5d %5d %3d  %10.4g %10.4g %10.4g %6.2f %8.2f %8.1f" % (
            n, M, N, K, s, fb, wb, a, (fb + wb) / a, ns / 1e3, (fb + wb) / ns))
        tot_b += fb + wb
        tot_a += a
        tot_t += ns
    lines += ["all %d launches: %.4g bytes against %.4g algorithmic (%.2fx), %.1f GB/s over %.1f us of kernel time"
              % (len(dt), tot_b, tot_a, tot_b / tot_a, tot_b / tot_t, tot_t / 1e3),
              "kernel source digest: %s" % source_digest([os.path.join(ROOT, "weight_only_quantized_qmm_amd", "csrc", f)
                                                          for f in ("qmm_w4a16_skinny.hip", "qmm_api.cpp",
                                                                    "qmm_launch.h", "qmm_device.h")])]
    print("\n".join(lines))


def summarize_decode_pmc(fetch_dir, write_dir, trace_dir, commands):
    """Text summary of the decode shapes' HBM traffic on both paths (the plan's small-M kernel
    and the matrix-vector kernel): FETCH_SIZE and WRITE_SIZE per launch (scaled by the copy
    kernel), the kernel-trace duration, the achieved HBM rate and the weight-read rate
    (packed weights + scale/bias over the launch's duration) as a fraction of 8 TB/s."""
    fetch = _counter_rows(fetch_dir, ["FETCH_SIZE"])["FETCH_SIZE"]
    write = _counter_rows(write_dir, ["WRITE_SIZE"])["WRITE_SIZE"]
    trace = _trace_durations(trace_dir)
    pick = lambda rows, key: [(k, v) for _, k, v in rows if key(k)]
    cf = [v for _, v in pick(fetch, lambda k: "calib_copy" in k)]
    cw = [v for _, v in pick(write, lambda k: "calib_copy" in k)]
    f_scale, w_scale = COPY_BYTES / (cf[0] * 1024.0), COPY_BYTES / (cw[0] * 1024.0)
    import qmm_synth as syn
    shapes = syn.decode_sweep()
    mine = lambda k: SMALL_KERNEL in k or GEMV_KERNEL in k
    # per shape and round: the plan's launch, then the matrix-vector launch (both unsplit here)
    df, dw, dt = [pick(rows, mine)[2 * len(shapes):] for rows in (fetch, write, trace)]
    lines = ["# HBM traffic of the decode shapes on %s and %s (%s) from rocprofv3 counters"
             % (SMALL_KERNEL, GEMV_KERNEL, DECODE_WORKLOAD), "commands:"] + ["  " + c for c in commands] + [
        "copy kernel: %d bytes read and written; FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB" % (COPY_BYTES, cf[0], cw[0]),
        "fetch scale: %.4f" % f_scale, "write scale: %.4f" % w_scale,
        "bytes = scaled FETCH + WRITE; algorithmic = packed weights + scale/bias + A + C; weight = packed weights +",
        "scale/bias; us = kernel-trace duration of the same launch (the merge of a split matrix-vector call not",
        "included); weight frac = weight bytes / us / 8 TB/s",
        "%-5s %2s %5s %5s %-7s %10s %10s %10s %6s %7s %8s %8s" % ("proj", "M", "N", "K", "path", "fetch B", "write B",
                                                                "algo B", "ratio", "us", "HBM GB/s", "wt frac")]
    for i, (n, M, N, K, _) in enumerate(shapes):
        wbytes = N * K // 2 + N * (K // 128) * 4
        a = algorithmic_bytes(M, N, K)
        for j, path in enumerate(("plan", "matvec")):
            (kf, fv), (_, wv), (kt, ns) = df[2 * i + j], dw[2 * i + j], dt[2 * i + j]
            assert (GEMV_KERNEL in kf) == (path == "matvec") and (GEMV_KERNEL in kt) == (path == "matvec"), (kf, kt)
            fb, wb = fv * 1024 * f_scale, wv * 1024 * w_scale
            lines.append("%-5s %2d %5d %5d %-7s %10.4g %10.4g %10.4g %6.2f %7.2f %8.1f %8.3f" % (
                n, M, N, K, path, fb, wb, a, (fb + wb) / a, ns / 1e3, (fb + wb) / ns, wbytes / ns / (HBM_PEAK / 1e9)))
    lines.append("kernel source digest: %s" % source_digest(
        [os.path.join(ROOT, "weight_only_quantized_qmm_amd", "csrc", f)
         for f in ("qmm_w4a16_skinny.hip", "qmm_gemv.hip", "qmm_api.cpp", "qmm_launch.h", "qmm_device.h")]))
    print("\n".join(lines))


def summarize_trace(trace_dir, commands, title, bench_avg_us=None):
    """Text summary of a rocprofv3 --kernel-trace --stats folder: calls and average duration
    of every kernel, the dominant kernel's variants combined."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % trace_dir)
    rows = [r for f in files for r in csv.DictReader(open(f))]

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "")
        return name.split("(")[0][:70]

    lines = ["# " + title, "commands:"] + ["  " + c for c in commands] + [
        "%-72s %7s %11s %9s" % ("kernel", "calls", "average_us", "pct")]
    dom_calls, dom_ns = 0, 0.0
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("%-72s %7d %11.3f %9.2f" % (short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                                 float(r["Percentage"])))
        if DOMINANT_KERNEL in r["Name"]:
            dom_calls += int(r["Calls"])
            dom_ns += float(r["TotalDurationNs"])
    if dom_calls:
        lines.append("%s, all variants together: %d calls, average %.3f us" % (DOMINANT_KERNEL, dom_calls,
                                                                             dom_ns / dom_calls / 1e3))
    if bench_avg_us:
        lines.append("bench.py's own figure in the same process (HIP events around graph replays): avg_launch_us = %s"
                     % bench_avg_us)
    print("\n".join(lines))


MIX_COUNTERS = (["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"],
                ["GRBM_GUI_ACTIVE", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS",
                 "SQ_VALU_MFMA_COEXEC_CYCLES"])


def summarize_mix(dir1, dir2, commands, n_xcc=8, n_cu=256):
    """Text summary of the dominant kernel's instruction mix and unit utilisation from two
    rocprofv3 --pmc passes (MIX_COUNTERS) over the large-M workload (pmc_run("large")).
    GRBM_GUI_ACTIVE is reported summed over the 8 XCDs, so the launch's active cycles are
    that sum / 8; per-SIMD counters are summed over the GPU's 1024 SIMDs, and the quad-cycle
    counters of a CU's 4 SIMDs (SQ_ACTIVE_INST_VALU) give the per-SIMD busy fraction as is."""
    a = _counter_rows(dir1, MIX_COUNTERS[0])
    b = _counter_rows(dir2, MIX_COUNTERS[1])
    import qmm_synth as syn
    shapes = [(n, M, N, K) for n, M, N, K, _ in syn.projection_sweep() if M > 128]

    def vals(rows, c):
        return [v for _, k, v in rows[c] if DOMINANT_KERNEL in k]

    simds = 4 * n_cu
    lines = ["# Instruction mix and unit utilisation of %s (%s) from rocprofv3 counters" % (
        DOMINANT_KERNEL, DOMINANT_WORKLOAD), "commands:"] + ["  " + c for c in commands] + [
        "active cycles = GRBM_GUI_ACTIVE / %d (summed over the XCDs); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /"
        " (active cycles x %d SIMDs);" % (n_xcc, simds),
        "VALU busy = SQ_ACTIVE_INST_VALU / (active cycles x %d CUs) (quad-cycles summed over a CU's 4 SIMDs: the"
        " per-SIMD fraction); LDS busy = SQ_LDS_IDX_ACTIVE / (active cycles x %d CUs);" % (n_cu, n_cu),
        "bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; co-issue = SQ_VALU_MFMA_COEXEC_CYCLES /"
        " SQ_VALU_MFMA_BUSY_CYCLES",
        "%-5s %6s %9s %9s %9s %9s %9s %8s %9s" % ("proj", "MFMA", "VALU/MFMA", "LDS/MFMA", "MFMA busy", "VALU busy",
                                                 "LDS busy", "bank cf", "co-issue")]
    rows = []
    for i, (n, M, N, K) in enumerate(shapes):
        g1, g2 = vals(a, "GRBM_GUI_ACTIVE")[i] / n_xcc, vals(b, "GRBM_GUI_ACTIVE")[i] / n_xcc
        mb = vals(a, "SQ_VALU_MFMA_BUSY_CYCLES")[i]
        va = vals(a, "SQ_ACTIVE_INST_VALU")[i]
        iv, im = vals(a, "SQ_INSTS_VALU")[i], vals(a, "SQ_INSTS_MFMA")[i]
        li, lb, il = vals(b, "SQ_LDS_IDX_ACTIVE")[i], vals(b, "SQ_LDS_BANK_CONFLICT")[i], vals(b, "SQ_INSTS_LDS")[i]
        co = vals(b, "SQ_VALU_MFMA_COEXEC_CYCLES")[i]
        r = dict(mfma=im, valu_per_mfma=(iv - im) / im, lds_per_mfma=il / im, mfma_busy=mb / (g1 * simds),
                 valu_busy=va / (g1 * n_cu), lds_busy=li / (g2 * n_cu), bank=lb / max(li, 1), coexec=co / max(mb, 1))
        rows.append(r)
        lines.append("%-5s %6.3g %9.2f %9.2f %9.3f %9.3f %9.3f %8.4f %9.3f" % (
            n, r["mfma"], r["valu_per_mfma"], r["lds_per_mfma"], r["mfma_busy"], r["valu_busy"], r["lds_busy"],
            r["bank"], r["coexec"]))
    mean = {k: sum(r[k] for r in rows) / len(rows) for k in rows[0]}
    lines += ["mean  %6.3g %9.2f %9.2f %9.3f %9.3f %9.3f %8.4f %9.3f" % (
        mean["mfma"], mean["valu_per_mfma"], mean["lds_per_mfma"], mean["mfma_busy"], mean["valu_busy"],
        mean["lds_busy"], mean["bank"], mean["coexec"]),
        "(SQ_INSTS_VALU counts the MFMA instructions too; VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA)",
        "kernel source digest: %s" % source_digest()]
    print("\n".join(lines))


LDS_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
                "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_LDS", "SQ_BUSY_CYCLES"]


def summarize_lds(d, commands, n_xcc=8, n_cu=256):
    """Text summary of one rocprofv3 --pmc pass (LDS_COUNTERS) over bench.py --dominant-only:
    LDS activity of the step-loop calibration kernels (whose LDS read bytes are known) beside
    that of the large-M kernel's variants, per kernel, summed over its dispatches."""
    import re
    rows = _counter_rows(d, LDS_COUNTERS)
    per = {}
    for c in LDS_COUNTERS:
        for disp, k, v in rows[c]:
            if "calib_step_kernel" not in k and DOMINANT_KERNEL not in k:
                continue
            name = re.sub(r"\(.*", "", k.replace("(anonymous namespace)::", "").replace("void ", "", 1))
            per.setdefault(name, {}).setdefault(c, {})
            per[name][c][disp] = per[name][c].get(disp, 0.0) + v
    lines = ["# LDS activity of the large-M kernel's step loop without global memory (calib_step_kernel<MI, NJ, "
             "LDS reads, dequantisation>: 8 waves of (32*MI) x (32*NJ) per CU, %d steps) and of %s, from rocprofv3 "
             "counters" % (STEP_LOOP_STEPS, DOMINANT_KERNEL), "commands:"] + ["  " + c for c in commands] + [
        "active cycles = GRBM_GUI_ACTIVE / %d; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x %d SIMDs); LDS active ="
        " SQ_LDS_IDX_ACTIVE / (cycles x %d CUs);" % (n_xcc, 4 * n_cu, n_cu),
        "LDS insts, FIFO full (data, command) and LDS waits (SQ_WAIT_INST_LDS) per CU and cycle; B/LDS-active cycle ="
        " the step loop's LDS read bytes (8 waves x MI x 1 KB per step) / SQ_LDS_IDX_ACTIVE",
        "%-52s %5s %9s %9s %9s %9s %9s %9s %11s" % ("kernel", "calls", "MFMA busy", "LDS act", "LDS inst", "data full",
                                                    "cmd full", "LDS wait", "B/LDS-cyc")]
    for name in sorted(per):
        c = {k: sum(v.values()) for k, v in per[name].items()}
        calls = len(per[name]["GRBM_GUI_ACTIVE"])
        cyc = c["GRBM_GUI_ACTIVE"] / n_xcc
        bpc = ""
        m = re.match(r"calib_step_kernel<(\d+), (\d+), (true|false), (true|false)>", name)
        if m and m.group(3) == "true" and c["SQ_LDS_IDX_ACTIVE"] > 0:
            nbytes = calls * n_cu * 8 * STEP_LOOP_STEPS * int(m.group(1)) * 1024
            bpc = "%.0f" % (nbytes / c["SQ_LDS_IDX_ACTIVE"])
        lines.append("%-52s %5d %9.3f %9.3f %9.4f %9.4f %9.4f %9.4f %11s" % (
            name, calls, c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 4 * n_cu), c["SQ_LDS_IDX_ACTIVE"] / (cyc * n_cu),
            c["SQ_INSTS_LDS"] / (cyc * n_cu), c["SQ_LDS_DATA_FIFO_FULL"] / (cyc * n_cu),
            c["SQ_LDS_CMD_FIFO_FULL"] / (cyc * n_cu), c["SQ_WAIT_INST_LDS"] / (cyc * n_cu), bpc))
    lines.append("kernel source digest: %s" % source_digest())
    print("\n".join(lines))


def summarize_pmc(fetch_dir, write_dir, commands):
    """Text summary of two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) over pmc_run()."""
    import csv
    import glob
    import qmm_synth as syn

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under %s" % d)
        rows = []
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                rows.append((int(r.get("Dispatch_Id") or len(rows)), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(rows)

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    pick = lambda rows, key: [v for _, k, v in rows if key in k]  # dispatch order
    cf, cw = pick(fetch, "calib_copy"), pick(write, "calib_copy")
    df, dw = pick(fetch, DOMINANT_KERNEL), pick(write, DOMINANT_KERNEL)
    f_scale = COPY_BYTES / (cf[0] * 1024.0)
    w_scale = COPY_BYTES / (cw[0] * 1024.0)
    shapes = [(n, M, N, K) for n, M, N, K, _ in syn.projection_sweep() if M > 128]
    alg = [algorithmic_bytes(M, N, K) for _, M, N, K in shapes]
    lines = ["# HBM traffic of %s (%s) from rocprofv3 counters" % (DOMINANT_KERNEL, DOMINANT_WORKLOAD),
             "commands:"] + ["  " + c for c in commands] + [
        "copy kernel: %d bytes read and written; FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB" % (COPY_BYTES, cf[0], cw[0]),
        "fetch scale: %.4f" % f_scale, "write scale: %.4f" % w_scale,
        "per launch (shape order %s):" % ", ".join(n for n, *_ in shapes)]
    tot = []
    for (n, M, N, K), a, fv, wv in zip(shapes, alg, df, dw):
        b = fv * 1024 * f_scale + wv * 1024 * w_scale
        tot.append(b)
        lines.append("  %-5s M=%d N=%d K=%d: fetch %.1f KiB, write %.1f KiB -> %.3e B scaled; algorithmic %.3e B (%.2fx)"
                     % (n, M, N, K, fv, wv, b, a, b / a))
    lines += ["kernel source digest: %s" % source_digest(),
              "hbm bytes per launch (scaled): %.6e" % (sum(tot) / len(tot)),
              "algorithmic bytes per launch: %.6e" % (sum(alg) / len(alg))]
    print("\n".join(lines))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=25.0, help="CPU-baseline sample budget")
    ap.add_argument("--no-per-shape", action="store_true")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--tables-out", default="bench_tables.json",
                    help="file that receives the per-shape and secondary tables (JSON)")
    ap.add_argument("--dominant-only", action="store_true",
                    help="only the dominant-kernel roofline measurement (the profiled command)")
    ap.add_argument("--pmc-run", nargs="?", const="large", choices=("large", "small", "decode"),
                    help="only the workload of the profiler counter passes (large: the M = 2048 first passes; "
                         "small: the small-M kernel's shapes)")
    ap.add_argument("--summarize-small-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="print the small-M kernel's traffic summary of two --pmc passes and a kernel trace")
    ap.add_argument("--summarize-decode-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="print the decode shapes' traffic summary (both paths) of two --pmc passes and a kernel trace")
    ap.add_argument("--summarize-lds", metavar="DIR",
                    help="print the LDS-activity summary of one --pmc pass (LDS_COUNTERS) over --dominant-only")
    ap.add_argument("--summarize-mix", nargs=2, metavar=("DIR1", "DIR2"),
                    help="print the dominant kernel's instruction-mix summary of two --pmc passes (MIX_COUNTERS)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "TITLE"),
                    help="print the kernel summary of a rocprofv3 --kernel-trace --stats folder")
    ap.add_argument("--bench-avg-us", default=None, help="bench.py's avg_launch_us of the traced run (recorded)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc output folders")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help="commands recorded in the traffic summary")
    return ap.parse_args()


class Shape:
    """Device buffers of one projection shape: R input sets, one output, one workspace."""

    def __init__(self, name, M, N, K, idx, sets, torch, syn, q, fmt=None, f32p=False):
        """fmt = (bits, group) runs qmm_wna16 (f32p: with fp32 partials); None runs qmm_w4a16_g128."""
        self.name, self.M, self.N, self.K, self.idx = name, M, N, K, idx
        self.q = q
        self.fmt, self.f32p = fmt, f32p
        self.plan = q.qmm_splitk_plan(M, N, K) if fmt is None else q.qmm_wna16_plan(fmt[0], fmt[1], M, N, K)
        self.s = self.plan.s
        d = syn.w4a16_weights(N, K, seed=2000 + idx) if fmt is None else syn.wq_inputs(fmt[0], fmt[1], 1, N, K,
                                                                                       seed=2000 + idx)
        A = syn.normal_bf16((M, K), seed=2500 + idx)

        def dev16(x):
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()

        base = (dev16(A), torch.from_numpy(d["Wq"].view("int32")).cuda(), dev16(d["scale"]), dev16(d["bias"]))
        self.sets = [base] + [tuple(t.clone() for t in base) for _ in range(sets - 1)]
        self.C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.ws = torch.empty(max(q.w4a16_workspace_bytes(M, N, self.s, f32p), 256), dtype=torch.uint8,
                              device="cuda")

    def call(self, r, s):
        """s = 0: the library's own plan (what a user gets); s >= 1: that explicit split."""
        A, W, S, B = self.sets[r % len(self.sets)]
        split = self.s if s == 0 else s
        ws, wsb = (self.ws, self.ws.numel()) if split > 1 else (None, 0)
        if self.fmt is None:
            self.q.qmm_w4a16_g128(A, W, S, B, self.C, self.M, self.N, self.K, s, ws, wsb)
        else:
            self.q.qmm_wna16(self.fmt[0], self.fmt[1], 1 if self.f32p else 0, A, W, S, B, self.C, self.M, self.N,
                             self.K, s, ws, wsb)

    def call_pass1(self, r):
        """The first pass alone of the plan's call (W4A16 g128): the matmul kernel's launch."""
        A, W, S, B = self.sets[r % len(self.sets)]
        ws, wsb = (self.ws, self.ws.numel()) if self.s > 1 else (None, 0)
        self.q.qmm_w4a16_g128_pass1(A, W, S, B, self.C, self.M, self.N, self.K, 0, ws, wsb)

    def set_bytes(self):
        return algorithmic_bytes(self.M, self.N, self.K, *(self.fmt or (4, 128)))

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


def time_graph(torch, g, reps=5, warm_s=0.03):
    """Median seconds of one replay, after replays for at least warm_s seconds: after an
    idle gap (buffer set-up on the host) the first few milliseconds of work run several
    per cent slower while the shader clock ramps up."""
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
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


def time_graphs_interleaved(torch, graphs, reps=7, warm_s=0.03):
    """Median seconds of one replay of each graph, the graphs replayed in turn (A, B, A, B, ...)
    after warm-up replays of all of them, so that a comparison between them sees the same
    clock and thermal state (timed one after the other, a few-per-cent drift between the
    two runs can reverse a few-per-cent difference)."""
    t0 = time.perf_counter()
    while True:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
    ts = [[] for _ in graphs]
    for _ in range(reps):
        for i, g in enumerate(graphs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            ts[i].append(e0.elapsed_time(e1) / 1e3)
    return [sorted(t)[len(t) // 2] for t in ts]


def per_shape(torch, syn, q, name, M, N, K, idx, fmt=None, f32p=False, unsplit=True):
    """Per-call seconds of the policy split and of the unsplit control over >= 1 GiB of rotation."""
    probe = Shape(name, M, N, K, idx, 1, torch, syn, q, fmt, f32p)
    R = max(8, min(1024, math.ceil(ROTATE_BYTES / probe.set_bytes())))
    probe.free()
    sh = Shape(name, M, N, K, idx, R, torch, syn, q, fmt, f32p)
    out = {}
    splits = [0, 1] if sh.s > 1 and unsplit else [0] if sh.s > 1 else [1]
    # the policy's split and the unsplit control replayed in turn (time_graphs_interleaved)
    gs = [graph_of(torch, lambda s=s: [sh.call(r, s) for r in range(R)]) for s in splits]
    for s, t in zip(splits, time_graphs_interleaved(torch, gs)):
        out[s] = t / R
    del gs
    if sh.s == 1:
        out[0] = out[1]
    out.setdefault(1, None)
    sh.free()
    torch.cuda.empty_cache()
    return sh, R, out


def cpu_baseline(syn, budget_s):
    """fp64 oracle on the host cores over the sweep, shape by shape, within a time budget;
    shapes the budget does not reach are extrapolated by multiply-add count."""
    import oracle

    cores = oracle.default_threads()
    shapes = syn.projection_sweep()
    # order: the small-M shapes, then the 2048-row shapes, each whole, until the budget is spent
    order = [sh for sh in shapes if sh[1] <= 128] + [sh for sh in shapes if sh[1] > 128]
    spent, sample, est_total = 0.0, [], 0.0
    done_macs, done_time = 0.0, 0.0
    for name, M, N, K, idx in order:
        if spent >= budget_s:
            break
        d = syn.w4a16_weights(N, K, seed=2000 + idx)
        A = syn.normal_bf16((M, K), seed=2500 + idx)
        t0 = time.perf_counter()
        oracle.qmm_w4a16(A, d["Wq"], d["scale"], d["bias"], M, N, K, s=1, nthreads=cores)
        dt = time.perf_counter() - t0
        spent += dt
        sample.append("%s M=%d" % (name, M))
        est_total += dt
        done_macs += M * N * K
        done_time += dt
    covered = {(s.split()[0], s.split()[1]) for s in sample}
    rate = done_time / done_macs  # seconds per MAC over the sample
    for name, M, N, K, idx in shapes:
        if (name, "M=%d" % M) not in covered:
            est_total += rate * M * N * K
    whole = len(sample) == len(shapes)
    # the 32 x 1024 x 2560 K-projection case on one thread (the all-core figure's reference point)
    M0, N0, K0 = 32, 1024, 2560
    d0 = syn.w4a16_inputs(M0, N0, K0, seed=0)
    t0 = time.perf_counter()
    oracle.qmm_w4a16(d0["A"], d0["Wq"], d0["scale"], d0["bias"], M0, N0, K0, s=1, nthreads=1)
    single = time.perf_counter() - t0
    return dict(value=est_total * 1e6,
                unit="us per sweep (35 projection matmuls%s)" % ("" if whole else ", extrapolated"),
                cores=cores, kind="oracle",
                sample="%s; %.1f s measured%s" % (
                    "the whole sweep, each shape once" if whole else ", ".join(sample), spent,
                    "" if whole else ", rest extrapolated by multiply-add count"),
                single_thread_32x1024x2560_us=round(single * 1e6, 1))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_commands)
        return
    if args.summarize_small_pmc:
        summarize_small_pmc(*args.summarize_small_pmc, args.pmc_commands)
        return
    if args.summarize_decode_pmc:
        summarize_decode_pmc(*args.summarize_decode_pmc, args.pmc_commands)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.pmc_commands, args.summarize_trace[1], args.bench_avg_us)
        return
    if args.summarize_mix:
        summarize_mix(*args.summarize_mix, args.pmc_commands)
        return
    if args.summarize_lds:
        summarize_lds(args.summarize_lds, args.pmc_commands)
        return
    if args.pmc_run:
        pmc_run(args.pmc_run)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
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

    if args.dominant_only:
        shapes = [Shape(n, M, N, K, i, 2, torch, syn, q) for n, M, N, K, i in sweep if M > 128]
        roof, calib = dominant_roofline(torch, shapes)
        print(json.dumps({"roofline": roof, "machine_floors": calib}), flush=True)
        return

    # ---- the timed step: the whole sweep, graph-replayed over two rotation sets
    shapes = [Shape(n, M, N, K, i, 2, torch, syn, q) for n, M, N, K, i in sweep]
    graphs = [graph_of(torch, lambda r=r: [sh.call(r, 0) for sh in shapes]) for r in range(2)]
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
        sh.call(0, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(3):
        for sh in shapes:
            sh.call(i, 0)
    torch.cuda.synchronize()
    eager_step_s = (time.perf_counter() - t0) / 3

    roof, calib = dominant_roofline(torch, shapes)
    del graphs
    for sh in shapes:
        sh.free()
    torch.cuda.empty_cache()

    # ---- per-shape table
    table = []
    if not args.no_per_shape:
        for n, M, N, K, i in sweep:
            sh, R, t = per_shape(torch, syn, q, n, M, N, K, i)
            r = roofline(M, N, K, t[0])
            # dispatches of one call: the matmul, plus the merge of the planes when the plan splits
            table.append(dict(name=n, M=M, N=N, K=K, s=sh.s, dispatches=1 if sh.s == 1 else 2,
                              full_tiles=sh.plan.full_tiles, us=round(t[0] * 1e6, 3),
                              us_unsplit=round(t[1] * 1e6, 3), speedup_vs_unsplit=round(t[1] / t[0], 3),
                              tflops=round(r["tflops"], 2), gbs=round(r["gbs"], 1), bound=r["bound"],
                              roof_us=round(r["t_roof_us"], 3), frac=round(r["frac"], 4), rotation_sets=R))
            progress("shape", table[-1], ("name", "M", "s", "dispatches", "us", "us_unsplit", "frac"))

    if table:
        # the practical floor of the HBM-bound shapes: a plain read of their algorithmic bytes
        floors = stream_floors(torch, [algorithmic_bytes(t["M"], t["N"], t["K"]) for t in table if t["M"] <= 128])
        for t in table:
            if t["M"] <= 128:
                f, c = floors[algorithmic_bytes(t["M"], t["N"], t["K"])]
                t["stream_floor_us"] = round(f * 1e6, 3)
                t["frac_of_stream_floor"] = round(f * 1e6 / t["us"], 4)
                t["chain_floor_us"] = round(c * 1e6, 3)
                t["frac_of_chain_floor"] = round(c * 1e6 / t["us"], 4)

    dense = decode = formats = attention = streamk = None
    if not args.no_per_shape:
        streamk = streamk_table(torch, syn, q, table)
        dense = dense_sweep(torch, syn, q)
        decode = decode_table(torch, syn, q)
        formats = formats_table(torch, syn, q)
        attention = attention_table(torch, q)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(syn, args.cpu_seconds)

    pol = q.policy_preset("QMM_POLICY_MI355X").as_dict()
    tables = {
        "shapes": table,
        "dense_bf16_splitk": dense,
        "decode": decode,
        "formats": formats,
        "decode_attention": attention,
        "streamk": streamk,
        "roofline_detail": roof,
        "machine_floors": calib,
        "policy": pol,
        "eager_us_per_step": round(eager_step_s * 1e6, 1),
        "wall_s_timed": round(wall, 4),
    }
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
                               "W4A16 g128, MI355X policy split", "shapes": len(sweep)},
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()
                     if k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "avg_launch_us",
                              "frac_of_measured_mfma_peak", "frac_of_step_loop")},
        "cpu_baseline": cpu,
    }
    line["roofline"]["kernel"] = "%s, first pass of the plan on the 7 M=2048 shapes" % DOMINANT_KERNEL
    if table:
        small = [t for t in table if t["M"] <= 128]
        line["summary"] = {
            "small_M_mean_frac": round(sum(t["frac"] for t in small) / len(small), 4),
            "small_M_mean_frac_of_stream_floor": round(sum(t["frac_of_stream_floor"] for t in small) / len(small), 4),
            "small_M_mean_frac_of_chain_floor": round(sum(t["frac_of_chain_floor"] for t in small) / len(small), 4),
            "M2048_mean_frac": round(sum(t["frac"] for t in table if t["M"] == 2048) / 7, 4),
            "split_never_slower": all(t["us"] <= t["us_unsplit"] for t in table),
            "sum_per_shape_us": round(sum(t["us"] for t in table), 2),
            "dispatches_per_sweep": sum(t["dispatches"] for t in table),
            "decode_best_us_max": (round(max(min(r["us"], r["gemv_us"]) for r in decode), 3) if decode else None),
            "dense_policy_us": dense["us"]["policy"] if dense else None,
        }
    if args.tables_out:
        d = os.path.dirname(args.tables_out)
        if d:
            os.makedirs(d, exist_ok=True)
        with open(args.tables_out, "w") as f:
            json.dump(dict(tables, headline=line), f, indent=1)
        line["tables"] = args.tables_out
    text = json.dumps(line, separators=(",", ":"))
    sys.stderr.flush()
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
