#!/usr/bin/env python3
"""Benchmark of the MX linear layer's hot path on one MI355X.

Headline workload: the W8A8 MXFP8 decode GEMV with 32x32 block scales,
M = 16 tokens, N = K = 7168.  One step is the whole hot path for one batch:
one mx_linear call on the bf16 activations, which quantizes them per token
(MXFP8, OCP rule) inside the GEMV kernel (one launch,
gemv_w8_fused_kernel).  Weights and codes are packed once
(load time, untimed); the step rotates over enough packed copies
(>= 512 MiB) that the 256 MB Infinity Cache cannot serve them, so every step
streams its weights from HBM.

value   = algorithmic weight + scale bytes per step / step time  (GB/s)
roofline.achieved = the same bytes / the dominant kernel's average duration
          per launch.  The step is one launch of the fused kernel, so this is
          the step's rate: `steps` launches replayed back to back from a HIP
          graph on the current stream, timed with HIP events (inter-launch
          gaps included, so a lower bound on the kernel's own rate).  The same
          GEMV on an activation pre-quantized into the T16 layout
          (gemv_w8_even_kernel) is timed the same way and reported as
          config.t16_kernel_ms.

The other workloads are timed the same way and reported under "secondary":
M = 1 and 4 of the same GEMV, the same GEMV fed by mx_quant_act's row-major
output, the A16W8 GEMVs (M = 1, N = 256, K = 512 and M = 8, N = 4096,
K = 1568), the A16W4 grouped MoE GEMV (E = 32, N = K = 3072, 16 tokens
top-8) and the prefill W8A8 GEMM (M = 4096, N = K = 7168, quantization +
GEMM per step; TFLOP/s against the 5.0 PFLOP/s fp8 peak).

Timing: each workload's steps are captured in a HIP graph.  The warm-up
graph (the requested number of steps) is replayed until at least
WARM_MS milliseconds of GPU work have run, so clocks have settled after the
idle seconds of input setup whatever --warmup says; then the graph of exactly
`steps` steps is replayed REPLAYS times, each replay bracketed by synchronize
and HIP events on the launch stream and queued behind about 1 ms of untimed
warm-up replays (so the stream is busy when the first event is reached), and
the median is reported.  The timed region includes the graph's own launch on
the GPU (about 9 us a replay on MI355X): at K = 20 short steps that adds some
0.4 us a step, at K = 200 a tenth of it.

cpu_baseline: the CPU oracle (fp64, OpenMP) computing the headline step on
the host cores: on every thread for about 8 s (`value`, `cores`), and on one
thread (`single_thread_value`), with the CPU model from /proc/cpuinfo.
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

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
CACHE_BYTES = 512 << 20          # rotate at least this many bytes of weights
WARM_MS = 200.0                  # least GPU time of warm-up replays per workload
REPLAYS = 5                      # timed replays of the steps graph; the median is reported


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2000 warm-up steps: about 24 ms of the headline step, enough for the
    # clocks to settle after the idle seconds of input setup (with 20, the
    # first timed graph measured about 3% slow)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--only", default=None,
                    help="run one workload only (gemv16, gemv1, gemv4, gemv16r, a16_c1, a16_c3, "
                         "moe, moe_block, gemm, gemv16_ceil, gemm_ceil)")
    ap.add_argument("--eager", action="store_true",
                    help="launch without HIP graphs (for hardware-counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 64 MiB device copy 20 times (counter calibration)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class GraphTimer:
    """Times steps captured in a HIP graph.

    Submitting one step from Python takes longer than the GPU needs to run
    it, so the steps are captured once (torch.cuda.CUDAGraph over the stream
    the library launches on) and the timed region is one replay of a graph
    holding exactly `steps` steps, bracketed by synchronize and HIP events.
    This is how a serving loop runs them (and how the pages tune their decode
    tiles: by graph replay latency)."""

    def __init__(self, torch):
        self.torch = torch

    def _graph(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            for i in range(n):
                fn(i)
        return g

    eager = False
    warm_ms = 0.0                      # the longest warm-up any workload took (ms of GPU time)

    def time(self, fn, steps, warmup):
        """ms per call of fn(i), over `steps` calls replayed back to back."""
        torch = self.torch
        for i in range(2):
            fn(i)                      # eager first calls (one-time setup)
        torch.cuda.synchronize()
        if GraphTimer.eager:           # counter runs: plain launches, rough timing
            t = time.perf_counter()
            for i in range(steps):
                fn(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t) * 1e3 / steps
        gw = self._graph(fn, max(warmup, 1))
        gt = self._graph(fn, steps)
        # warm-up: the requested steps, replayed until WARM_MS of GPU time
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        warm, replays_warm = 0.0, 0
        while True:
            e0.record()
            gw.replay()
            e1.record()
            torch.cuda.synchronize()
            warm += e0.elapsed_time(e1)
            replays_warm += 1
            if warm >= WARM_MS:
                break
        GraphTimer.warm_ms = max(GraphTimer.warm_ms, warm)
        # Each timed replay is queued behind about 1 ms of untimed warm-up
        # replays, so the GPU is busy (and its clocks up) when the first event
        # is reached.  The graph's own launch on the GPU, about 9 us a replay,
        # stays inside the timed region: at K = 20 short steps some 0.4 us a
        # step.
        cover = max(1, int(-(-1.0 // (warm / replays_warm))))
        times = []
        for _ in range(REPLAYS):
            torch.cuda.synchronize()
            for _ in range(cover):
                gw.replay()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            gt.replay()
            t1.record()
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) / steps)
        times.sort()
        return times[len(times) // 2]

    def run(self, step, kernel, steps, warmup):
        """(ms per step, ms per launch of the dominant kernel alone)."""
        ms_step = self.time(lambda i: (step(i), kernel(i)), steps, warmup)
        ms_kernel = self.time(kernel, steps, warmup)
        return ms_step, ms_kernel


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "microscaling_quantized_linear_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, sha):
    """HBM bytes per launch measured by rocprofv3 counters for this workload,
    from profiles/hbm_traffic.md, if the kernel source is unchanged since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for m in re.finditer(r"<!--traffic (\{.*?\})-->", open(path).read()):
        rec = json.loads(m.group(1))
        if rec.get("workload") == workload and rec.get("source_sha") == sha:
            return rec.get("bytes_per_launch")
    return None


# ---------------------------------------------------------------- workloads

def setup_dense(torch, mx, g, wl, cid, M, rotate=True):
    d = wl.linear_inputs(cid, M=M)
    N, K = d["N"], d["K"]
    wp, cp = g.pack(d["elem"], d["layout"], 1, N, K, d["w"], d["codes"])
    per = wp.numel() + cp.numel()
    copies = max(1, -(-CACHE_BYTES // per)) if rotate else 1
    copies = min(copies, 4096)
    wps = [wp] + [wp.clone() for _ in range(copies - 1)]
    cps = [cp] + [cp.clone() for _ in range(copies - 1)]
    return d, wps, cps


def bench_w8a8_gemv(torch, mx, g, wl, M, steps, warmup, rowmajor=False, rule=None):
    """W8A8 decode GEMV, N = K = 7168, 32x32 block codes.

    Default: one mx_linear call per step with the activation quantized inside
    the call (per token, OCP rule, into the T16 layout), then the GEMV; the
    kernel-only timing runs the same GEMV on a pre-quantized T16 activation.
    rowmajor: mx_quant_act (row-major output) then mx_linear on it.
    rule: the activation scale rule (default OCP; MX_RULE_CEIL448 is the
    pages' ceil(log2(amax / 448)) rule, reported as its own line)."""
    rule = mx.MX_RULE_OCP if rule is None else rule
    d, wps, cps = setup_dense(torch, mx, g, wl, 2, M)
    N, K = d["N"], d["K"]
    x = g.dev(d["x"][:M])
    y = torch.empty((M, N), dtype=torch.int16, device=g.DEV)
    nc = len(wps)
    E, L, A8, T16 = mx.MX_E4M3, mx.MX_SCALE_BLK32, mx.MX_ACT_MXFP8, mx.MX_ACT_MXFP8_T16
    if rowmajor:
        xq = torch.empty((M, K), dtype=torch.uint8, device=g.DEV)
        xc = torch.empty((M, K // 32), dtype=torch.uint8, device=g.DEV)

        def step(i):
            mx.mx_quant_act(M, K, x, K, xq, K, xc, K // 32, mx.MX_RULE_OCP)

        def kernel(i):
            mx.mx_linear(E, L, N, K, wps[i % nc], cps[i % nc], M, A8, mx.MX_RULE_OCP, None, 0,
                         xq, K, xc, K // 32, None, y, N, None, 0)

        ms_step, ms_k = GraphTimer(torch).run(step, kernel, steps, warmup)
        how = "mx_quant_act (row-major) + mx_linear on it"
        kname = "gemv_w8_kernel (BLK32, row-major activations)"
    else:
        need = mx.mx_linear_workspace(E, L, N, K, M, A8, 0)
        ws = torch.empty(need, dtype=torch.uint8, device=g.DEV)
        qb, cb = mx.mx_act_t16_sizes(M, K)
        xq = torch.empty(qb, dtype=torch.uint8, device=g.DEV)
        xc = torch.empty(cb, dtype=torch.uint8, device=g.DEV)
        mx.mx_quant_act_t16(M, K, x, K, xq, xc, mx.MX_RULE_OCP)

        def step(i):
            mx.mx_linear(E, L, N, K, wps[i % nc], cps[i % nc], M, A8, rule, x, K,
                         None, 0, None, 0, None, y, N, ws, need)

        def kernel(i):
            mx.mx_linear(E, L, N, K, wps[i % nc], cps[i % nc], M, T16, mx.MX_RULE_OCP, None, 0,
                         xq, 0, xc, 0, None, y, N, None, 0)

        timer = GraphTimer(torch)
        ms_step = timer.time(step, steps, warmup)
        ms_t16 = timer.time(kernel, steps, warmup)
        fused = need == 0
        # with the quantization inside the GEMV the step is one launch of
        # gemv_w8_fused_kernel: the step's time is that kernel's time
        ms_k = ms_step if fused else ms_t16
        rname = "OCP rule" if rule == mx.MX_RULE_OCP else "ceil(log2(amax/448)) rule"
        how = (f"mx_linear with MXFP8 quantization ({rname}) inside the GEMV: one launch"
               if fused else f"mx_linear with in-call MXFP8 quantization ({rname}) then the GEMV")
        kname = ("gemv_w8_fused_kernel (BLK32, per-token quantization inside)" if fused
                 else "gemv_w8_even_kernel (BLK32, T16 activations)")
    alg = N * K + (N // 32) * (K // 32)
    out = dict(workload=f"mxfp8_w8a8_gemv_M{M}_N{N}_K{K}_blk32" + ("_rowmajor" if rowmajor else "")
               + ("_ceil448" if rule != mx.MX_RULE_OCP else ""),
               M=M, N=N, K=K, bytes_per_step=alg, weight_copies=nc, ms_per_step=ms_step,
               ms_kernel=ms_k, value=alg / (ms_step * 1e-3) / 1e9, unit="GB/s",
               kernel_gbs=alg / (ms_k * 1e-3) / 1e9, kernel=kname, step=how,
               src="mx_gemv_w8.hip")
    if not rowmajor:
        # the same GEMV on an activation pre-quantized into the T16 layout
        out["t16_kernel"] = "gemv_w8_even_kernel (BLK32, T16 activations)"
        out["t16_kernel_ms"] = ms_t16
        out["t16_kernel_gbs"] = alg / (ms_t16 * 1e-3) / 1e9
    return out


def bench_a16_gemv(torch, mx, g, wl, cid, steps, warmup):
    d, wps, cps = setup_dense(torch, mx, g, wl, cid, None)
    N, K, M = d["N"], d["K"], d["M"]
    x = g.dev(d["x"])
    y = torch.empty((M, N), dtype=torch.int16, device=g.DEV)
    nc = len(wps)

    def kernel(i):
        mx.mx_linear(mx.MX_E4M3, mx.MX_SCALE_ROW32, N, K, wps[i % nc], cps[i % nc], M,
                     mx.MX_ACT_BF16, 0, x, K, None, 0, None, 0, None, y, N, None, 0)

    ms_k = GraphTimer(torch).time(kernel, steps, warmup)
    ms_step = ms_k
    alg = N * K + N * (K // 32)
    return dict(workload=wl.WORKLOADS[cid]["name"], M=M, N=N, K=K, bytes_per_step=alg,
                weight_copies=nc, ms_per_step=ms_step, ms_kernel=ms_k,
                value=alg / (ms_step * 1e-3) / 1e9, unit="GB/s",
                kernel_gbs=alg / (ms_k * 1e-3) / 1e9, kernel="gemv_kernel (A16W8, ROW32)",
                src="mx_gemv.hip")


def bench_moe(torch, mx, g, wl, steps, warmup):
    import numpy as np
    d = wl.moe_inputs(4)
    E, N, K, T, topk = d["E"], d["N"], d["K"], d["T"], d["topk"]
    wp, cp = g.pack(1, 0, E, N, K, d["w"], d["codes"])
    per = wp.numel() + cp.numel()
    nc = max(1, -(-CACHE_BYTES // per))
    wps = [wp] + [wp.clone() for _ in range(nc - 1)]
    cps = [cp] + [cp.clone() for _ in range(nc - 1)]
    x = g.dev(d["x"])
    ids = g.dev(d["ids"])
    y = torch.empty((T, topk, N), dtype=torch.int16, device=g.DEV)

    def kernel(i):
        mx.mx_moe_linear(1, E, N, K, wps[i % nc], cps[i % nc], T, topk, x, K, ids, None, y, None,
                         0)

    ms_k = GraphTimer(torch).time(kernel, steps, warmup)
    ms_step = ms_k
    touched = len(np.unique(d["ids"]))
    alg = touched * (N * K // 2 + N * (K // 32))
    return dict(workload=wl.WORKLOADS[4]["name"], E=E, N=N, K=K, T=T, topk=topk,
                experts_touched=touched, bytes_per_step=alg, weight_copies=nc,
                ms_per_step=ms_step, ms_kernel=ms_k, value=alg / (ms_step * 1e-3) / 1e9,
                unit="GB/s", kernel_gbs=alg / (ms_k * 1e-3) / 1e9,
                kernel="gemv_kernel (A16W4, MoE)", src="mx_gemv.hip")


def bench_moe_block(torch, mx, g, wl, steps, warmup):
    """MoE block at the MoE decode shape (E = 32 experts, hidden 3072,
    intermediate 1536, T = 16 tokens, top-8, A16W4): per step the up-gate GEMV
    over interleaved gate/up rows with the SiLU product fused, then the down
    projection on the per-slot hidden rows with the weighted combine."""
    import numpy as np
    d13 = wl.moe_inputs(4)                                  # w13 rows: [E, 2 inter, K]
    E, N13, Hd, T, topk = d13["E"], d13["N"], d13["K"], d13["T"], d13["topk"]
    inter = N13 // 2
    d2 = wl.moe_inputs(4, N=Hd, K=inter, seed=1)            # w2: [E, hidden, inter]
    w13p, c13p = g.pack(1, 0, E, N13, Hd, d13["w"], d13["codes"])
    w2p, c2p = g.pack(1, 0, E, Hd, inter, d2["w"], d2["codes"])
    per = w13p.numel() + c13p.numel() + w2p.numel() + c2p.numel()
    nc = max(1, -(-CACHE_BYTES // per))
    sets = [(w13p, c13p, w2p, c2p)] + [(w13p.clone(), c13p.clone(), w2p.clone(), c2p.clone())
                                       for _ in range(nc - 1)]
    x = g.dev(d13["x"])
    ids = g.dev(d13["ids"])
    wts = g.dev(d13["weights"])
    h = torch.empty((T * topk, inter), dtype=torch.int16, device=g.DEV)
    y = torch.empty((T, Hd), dtype=torch.int16, device=g.DEV)
    need = mx.mx_moe_workspace(1, E, Hd, inter, T, topk, True)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=g.DEV)

    def gate_up(i):
        a, b, _, _ = sets[i % nc]
        mx.mx_moe_gate_up(1, E, inter, Hd, a, b, T, topk, x, Hd, ids, h, inter)

    def step(i):
        gate_up(i)
        _, _, a, b = sets[i % nc]
        mx.mx_moe_down(1, E, Hd, inter, a, b, T, topk, h, inter, ids, wts, y, ws, need)

    timer = GraphTimer(torch)
    ms_step = timer.time(step, steps, warmup)
    ms_k = timer.time(gate_up, steps, warmup)
    touched = len(np.unique(d13["ids"]))
    b13 = touched * (N13 * Hd // 2 + N13 * (Hd // 32))
    b2 = touched * (Hd * inter // 2 + Hd * (inter // 32))
    return dict(workload="mxfp4_a16w4_moe_block_E32_H3072_I1536_T16_top8", E=E, hidden=Hd,
                inter=inter, T=T, topk=topk, experts_touched=touched, bytes_per_step=b13 + b2,
                bytes_gate_up=b13, weight_copies=nc, ms_per_step=ms_step, ms_kernel=ms_k,
                value=(b13 + b2) / (ms_step * 1e-3) / 1e9, unit="GB/s",
                kernel_gbs=b13 / (ms_k * 1e-3) / 1e9,
                kernel="gemv_kernel (A16W4, MoE up-gate with SiLU product)",
                step="mx_moe_gate_up + mx_moe_down (combine)", src="mx_gemv.hip")


def bench_gemm(torch, mx, g, wl, steps, warmup, rule=None):
    """Prefill W8A8 GEMM, M = 4096, N = K = 7168: per step one mx_linear with
    the activation quantized inside the call (T16 layout) then the GEMM; the
    kernel-only timing runs the GEMM on a pre-quantized T16 activation.
    rule: the activation scale rule of the step (default OCP)."""
    rule = mx.MX_RULE_OCP if rule is None else rule
    d = wl.linear_inputs(5)
    N, K, M = d["N"], d["K"], d["M"]
    wp, cp = g.pack(0, 1, 1, N, K, d["w"], d["codes"])
    x = g.dev(d["x"])
    y = torch.empty((M, N), dtype=torch.int16, device=g.DEV)
    need = mx.mx_linear_workspace(0, 1, N, K, M, mx.MX_ACT_MXFP8, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=g.DEV)
    qb, cb = mx.mx_act_t16_sizes(M, K)
    xq = torch.empty(qb, dtype=torch.uint8, device=g.DEV)
    xc = torch.empty(cb, dtype=torch.uint8, device=g.DEV)
    mx.mx_quant_act_t16(M, K, x, K, xq, xc, mx.MX_RULE_OCP)

    def step(i):
        mx.mx_linear(0, 1, N, K, wp, cp, M, mx.MX_ACT_MXFP8, rule, x, K, None, 0,
                     None, 0, None, y, N, ws, need)

    def kernel(i):
        mx.mx_linear(0, 1, N, K, wp, cp, M, mx.MX_ACT_MXFP8_T16, 0, None, 0, xq, 0, xc, 0,
                     None, y, N, None, 0)

    timer = GraphTimer(torch)
    ms_step = timer.time(step, steps, warmup)
    ms_k = timer.time(kernel, steps, warmup)
    flop = 2.0 * M * N * K
    rname = "OCP rule" if rule == mx.MX_RULE_OCP else "ceil(log2(amax/448)) rule"
    return dict(workload=wl.WORKLOADS[5]["name"] + ("_ceil448" if rule != mx.MX_RULE_OCP else ""),
                M=M, N=N, K=K, flop_per_step=flop,
                ms_per_step=ms_step, ms_kernel=ms_k, value=flop / (ms_step * 1e-3) / 1e12,
                unit="TFLOP/s", kernel_tflops=flop / (ms_k * 1e-3) / 1e12,
                kernel="gemm_w8a8_kernel (BLK32, T16 activations)",
                step=f"mx_linear with in-call MXFP8 quantization ({rname})", src="mx_gemm.hip")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl):
    """The oracle, as it stands, computing the headline step (per-token
    quantization of M = 16 rows, then the fp64 linear with N = K = 7168) on
    every host thread for about 8 s, then on one thread (a few runs)."""
    import oracle
    d = wl.linear_inputs(2, M=16)
    N, K = d["N"], d["K"]
    alg = N * K + (N // 32) * (K // 32)

    def run(budget_s, max_runs):
        runs, t_total = 0, 0.0
        while (t_total < budget_s or runs < 1) and runs < max_runs:
            t = time.perf_counter()
            xq, xc = oracle.quant_act(d["x"], oracle.RULE_OCP)
            oracle.linear(0, 1, N, K, d["w"], d["codes"], 16, oracle.ACT_MXFP8, xq=xq, xcodes=xc)
            t_total += time.perf_counter() - t
            runs += 1
        return runs, t_total / runs

    cores = oracle.threads()
    runs, sec = run(8.0, 2000)
    prev = oracle.set_threads(1)
    try:
        runs1, sec1 = run(4.0, 8)
    finally:
        oracle.set_threads(prev)
    return {"value": alg / sec / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the full headline step (M=16, N=K=7168: quant + fp64 linear), "
                      f"{runs} runs on {cores} threads, {sec:.3f} s each; "
                      f"{runs1} runs on 1 thread, {sec1:.2f} s each",
            "single_thread_value": alg / sec1 / 1e9, "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "a single-GPU kernel library and measures no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import microscaling_quantized_linear_amd as mx
    from microscaling_quantized_linear_amd import workloads as wl
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import mxgpu as g

    mx.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a gfx950 GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    if args.copy_calibration:
        a = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(20):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel(), "launches": 20}))
        return
    GraphTimer.eager = args.eager

    only = args.only
    want = (lambda n: only is None or only == n)
    head = None
    sec = []
    if want("gemv16"):
        log("headline: W8A8 GEMV M=16 N=K=7168")
        head = bench_w8a8_gemv(torch, mx, g, wl, 16, K, W)
        log(json.dumps(head))
    if not args.no_secondary:
        if want("gemv1"):
            sec.append(bench_w8a8_gemv(torch, mx, g, wl, 1, K, W)); log(json.dumps(sec[-1]))
        if want("gemv16r"):
            sec.append(bench_w8a8_gemv(torch, mx, g, wl, 16, K, W, rowmajor=True))
            log(json.dumps(sec[-1]))
        if want("gemv4"):
            sec.append(bench_w8a8_gemv(torch, mx, g, wl, 4, K, W)); log(json.dumps(sec[-1]))
        if want("a16_c1"):
            sec.append(bench_a16_gemv(torch, mx, g, wl, 1, K, W)); log(json.dumps(sec[-1]))
        if want("a16_c3"):
            sec.append(bench_a16_gemv(torch, mx, g, wl, 3, K, W)); log(json.dumps(sec[-1]))
        if want("moe"):
            sec.append(bench_moe(torch, mx, g, wl, K, W)); log(json.dumps(sec[-1]))
        if want("moe_block"):
            sec.append(bench_moe_block(torch, mx, g, wl, K, W)); log(json.dumps(sec[-1]))
        if want("gemm"):
            sec.append(bench_gemm(torch, mx, g, wl, max(10, K // 4), max(3, W // 4)))
            log(json.dumps(sec[-1]))
        # the pages' own scale rule, ceil(log2(amax / 448)), on the same two steps
        if want("gemv16_ceil"):
            sec.append(bench_w8a8_gemv(torch, mx, g, wl, 16, K, W, rule=mx.MX_RULE_CEIL448))
            log(json.dumps(sec[-1]))
        if want("gemm_ceil"):
            sec.append(bench_gemm(torch, mx, g, wl, max(10, K // 4), max(3, W // 4),
                                  rule=mx.MX_RULE_CEIL448))
            log(json.dumps(sec[-1]))
    if head is None:
        head = sec[0]
    for s in sec:
        if s["unit"] == "GB/s":
            s["roofline_frac"] = round(s["kernel_gbs"] / HBM_PEAK_GBS, 4)
        else:
            s["roofline_frac"] = round(s["kernel_tflops"] / FP8_PEAK_TFLOPS, 4)

    for s in [head] + sec:
        s["traffic"] = recorded_traffic(s["workload"], source_sha(s["src"], "mx_device.h"))
    if head["unit"] == "GB/s":
        roof = {"bound": "hbm", "achieved": round(head["kernel_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["kernel_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": head["traffic"]}
    else:
        roof = {"bound": "mfma", "achieved": round(head["kernel_tflops"], 1),
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(head["kernel_tflops"] / FP8_PEAK_TFLOPS, 4),
                "traffic": head["traffic"]}
    cpu = None if args.no_cpu else cpu_baseline(wl)
    out = {
        "metric": "achieved HBM GB/s (weights+scales) for M≤16 MX GEMV; TFLOP/s for M=4096 GEMM",
        "value": round(head["value"], 1),
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "warmup_ms": round(GraphTimer.warm_ms, 1),
        "timed_replays": REPLAYS,

        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8",
        "data": "synthetic",
        "config": {"workload": head["workload"], "M": head.get("M"), "N": head.get("N"),
                   "K": head.get("K"), "step": head.get("step"),
                   "weight_copies_rotated": head.get("weight_copies"),
                   "kernel": head.get("kernel"),
                   "kernel_ms": round(head["ms_kernel"], 5),
                   "t16_kernel_ms": (round(head["t16_kernel_ms"], 5)
                                     if "t16_kernel_ms" in head else None)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in s.items()}
                      for s in sec],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
