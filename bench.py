#!/usr/bin/env python3
"""Benchmark of the MHLA forward on one MI355X.

One step = one mhla_forward call: the whole hot path (block summaries,
multi-head mixing, readout) over one batch of seeded synthetic input that is
already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload video] [--path auto]

The default workload is the video-latent case (B1 H24 N32768 as an 8x64x64
grid of 1x8x8 blocks, so M=512; d64; elu+1), the largest configuration and
the one where the M^2 d^2 mixing term dominates.  The other workloads (tiny,
deit_t, dit_xl2, hires, lm_causal) can be selected for study.

Timing: the K steps are enqueued back to back from arguments marshalled once
(no Python checks inside the loop) and bracketed by HIP events on the launch
stream; `ms_per_step` and `value` come from that bracket.  A second run of at
least 50 calls records events around every kernel launch of every call
(mhla_forward_profiled): the median call time and each kernel's median launch
time come from it, and the roofline object is that of the kernel with the
largest median time.

  python bench.py --copy-mb 256

times a plain device copy of that size instead (the reference kernel for
scaling the HBM byte counters of a profiler run), and

  python bench.py --library-gemm --workload video

times the vendor BLAS on the large-M mixing GEMM's shape.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published
METRIC = "MHLA fwd tokens/s per GPU and % of bf16 MFMA / HBM roofline"
MIN_PROFILED_CALLS = 50


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="video")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "generic", "fused", "pairs", "blocked", "columns"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single-core", action="store_true",
                    help="skip the single-core oracle timings of the four smaller workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="time a plain device copy of this many MB instead")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor BLAS (torch.bmm, bf16) on the workload's mixing GEMM "
                         "shape, H x [M x M] @ [M x d*d], instead: a reference for the large-M "
                         "mixing kernel")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (mhla_backward) instead of the forward")
    ap.add_argument("--decode", action="store_true",
                    help="time token-by-token causal inference (mhla_decode_step) over the "
                         "workload's sequence instead (1-D chunked workloads, e.g. lm_causal)")
    return ap.parse_args()


class HipEvents:
    """A pool of timing events of the HIP runtime (the same runtime torch
    uses), created once; elapsed() reads the time between two of them."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.ev = []


def copy_bench(args):
    import torch
    n = args.copy_mb * 1000 * 1000 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"copy_bytes_each_way": n * 4, "steps": args.steps, "ms_per_copy": ms,
                      "GBs_read_plus_write": 2 * n * 4 / (ms / 1e3) / 1e9}), flush=True)
    return 0


def kernel_work(name, wl, path_name):
    """(bytes, flops) that one launch of kernel `name` must move and compute on
    workload wl, by design: its own inputs read once and outputs written once
    (the block summary tables S and S~ count for the kernels that write and
    read them), and the method's flops of its step (summaries and readout
    2*N*d^2, mixing 2*M^2*d^2 per slice).  Single-kernel paths move exactly
    the algorithmic bytes of the call."""
    S = wl.B * wl.H
    T = S * wl.N * wl.d * wl.elt_bytes                 # one of Q, K, V, Y
    ws_elt = 4 if path_name == "generic" else 2
    E = S * wl.M * (wl.d * wl.d + wl.d) * ws_elt        # one summary table
    Wb = wl.H * wl.M * wl.M * 4
    f_side = 2 * wl.N * wl.d * wl.d * S                 # summaries or readout
    f_mix = 2 * wl.M * wl.M * wl.d * wl.d * S
    if name in ("k_fused", "k_pairs", "k_cols", "k_generic_one"):
        return wl.algorithmic_bytes(), wl.algorithmic_flops()
    if name.startswith("k_summary"):
        return 2 * T + E, f_side
    Ed = S * wl.M * wl.d * wl.d * ws_elt                # the d*d entries of a table
    Z = S * wl.M * wl.d * ws_elt                        # the z entries of a table
    if name == "k_mix_coef_t":
        return Wb + Wb // 2, 0
    if name == "k_mix_prep":                            # W -> bf16 coefficients, z~ = W z
        return Wb + Wb // 2 + 2 * Z, 2 * wl.M * wl.M * wl.d * S
    if name == "k_mix_big" and wl.M >= 256:
        return 2 * Ed + Wb // 2, f_mix                  # the d*d entries, bf16 coefficients
    if name == "k_mix_big":
        return 2 * E + Wb // 2, f_mix
    if name.startswith("k_mix"):
        return 2 * E + Wb, f_mix
    if name == "k_readout_causal":
        return 4 * T + E, f_side + 2 * wl.N * wl.nb * wl.d * S
    if name.startswith("k_readout"):
        return 2 * T + E, f_side
    return 0, 0


def roofline_entry(nbytes, flops, ms, fp32=False):
    """Fractions of the HBM and the matrix-core (or fp32 vector) peak for one
    kernel or call; the binding one is the larger."""
    gbs = nbytes / (ms / 1e3) / 1e9
    peak_f = FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS
    tfs = flops / (ms / 1e3) / 1e12
    if gbs / HBM_PEAK_GBS >= tfs / peak_f:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        r = {"bound": "alu" if fp32 else "mfma", "achieved": round(tfs, 1), "peak": peak_f,
             "unit": "TFLOP/s", "frac": round(tfs / peak_f, 4)}
    r.update({"hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "flop_frac": round(tfs / peak_f, 4)})
    return r


def library_gemm_bench(args):
    """The mixing step S~ = W S of one head is a plain GEMM of shape
    [M x M] @ [M x d*d] (bf16 operands, fp32 accumulation); this times the
    vendor library (torch.bmm -> hipBLASLt / rocBLAS) on it, batched over the
    heads, as a reference for the large-M mixing kernel."""
    import torch
    from mhla_inputs import WORKLOADS
    wl = WORKLOADS[args.workload]
    g = torch.Generator(device="cpu").manual_seed(0)
    S = wl.B * wl.H
    A = (torch.randn(S, wl.M, wl.M, generator=g) * 0.05).to(torch.bfloat16).cuda().contiguous()
    Bm = torch.randn(S, wl.M, wl.d * wl.d, generator=g).to(torch.bfloat16).cuda().contiguous()
    C = torch.empty(S, wl.M, wl.d * wl.d, dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        torch.bmm(A, Bm, out=C)
    torch.cuda.synchronize()
    ts = []
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.bmm(A, Bm, out=C)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = statistics.median(ts)
    flops = 2.0 * S * wl.M * wl.M * wl.d * wl.d
    print(json.dumps({"library_gemm": "torch.bmm bf16", "workload": wl.name,
                      "shape": [S, wl.M, wl.M, wl.d * wl.d], "median_us": round(ms * 1e3, 2),
                      "TFLOPs": round(flops / (ms / 1e3) / 1e12, 1),
                      "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}),
          flush=True)
    return 0


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the (batch, head) slices would shard across GPUs with no communication, but "
              "that launcher is not part of this build)" % args.gpus, file=sys.stderr)
        return 2
    if args.copy_mb:
        return copy_bench(args)
    if args.library_gemm:
        return library_gemm_bench(args)
    if args.backward:
        return backward_bench(args)
    if args.decode:
        return decode_bench(args)

    import torch
    import token_level_head_mhla_amd as m
    from mhla_inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    path = {"auto": m.MHLA_PATH_AUTO, "generic": m.MHLA_PATH_GENERIC,
            "fused": m.MHLA_PATH_FUSED, "pairs": m.MHLA_PATH_PAIRS,
            "blocked": m.MHLA_PATH_BLOCKED, "columns": m.MHLA_PATH_COLUMNS}[args.path]
    shape = (wl.grid, wl.block)
    if path == m.MHLA_PATH_AUTO:
        path = m.mhla_plan_ex(wl.B, wl.H, wl.N, wl.d, m.BlockShape.make(*shape), wl.phi,
                              wl.dtype, wl.flags)
    path_name = {1: "generic", 2: "fused", 3: "pairs", 4: "blocked", 5: "columns"}[path]

    inp = make_inputs(wl)

    def dev(x):
        if wl.dtype == 1:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()  # the stream the library launches on
    call = m.PreparedForward(q, k, v, w, out, shape, wl.phi, wl.flags, path, stream=stream)

    for _ in range(args.warmup):
        call.call()
    torch.cuda.synchronize()
    # Per-call and per-launch times first (they also bring the clocks up):
    # >= 50 profiled calls, each with its own events, enqueued back to back.
    nprof = max(args.steps, MIN_PROFILED_CALLS)
    per = m.MHLA_MAX_LAUNCHES + 1
    pool = HipEvents(per * nprof)
    names = None
    for c in range(nprof):
        names = call.profiled(pool.ev[c * per:(c + 1) * per])
    torch.cuda.synchronize()
    nl = len(names)
    launch_ms = np.array([[pool.elapsed(pool.ev[c * per + j], pool.ev[c * per + j + 1])
                           for j in range(nl)] for c in range(nprof)])
    call_ms = np.array([pool.elapsed(pool.ev[c * per], pool.ev[c * per + nl])
                        for c in range(nprof)])
    pool.close()
    # K steps back to back, bracketed by HIP events on the launch stream; the
    # host's enqueue time is measured alongside.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    h0 = time.perf_counter()
    for _ in range(args.steps):
        call.call()
    host_s = time.perf_counter() - h0
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens = wl.B * wl.N
    value = tokens / (ms / 1e3)

    prof_call = float(np.median(call_ms))
    kernels = []
    for j, nm in enumerate(names):
        kb, kf = kernel_work(nm, wl, path_name)
        # A call of one launch is timed by the bracket of K back-to-back calls
        # (the events around each profiled launch add a few microseconds,
        # which matters for kernels this short); several launches per call
        # are timed by the events between them.
        t = ms if nl == 1 else float(np.median(launch_ms[:, j]))
        e = {"kernel": nm, "median_us": round(t * 1e3, 3), "bytes": kb, "flops": kf,
             "profiled_median_us": round(float(np.median(launch_ms[:, j])) * 1e3, 3)}
        e.update(roofline_entry(kb, kf, t, fp32=(path_name == "generic")))
        kernels.append(e)
    dom = max(range(nl), key=lambda j: kernels[j]["median_us"])
    dk = kernels[dom]
    # the roofline of the dominant kernel: its algorithmic work per launch over
    # its average launch duration (the figure a profiler's kernel statistics give)
    avg_t = ms if nl == 1 else float(np.mean(launch_ms[:, dom]))
    dom_rl = roofline_entry(dk["bytes"], dk["flops"], avg_t, fp32=(path_name == "generic"))
    roofline = {k_: dom_rl[k_] for k_ in ("bound", "achieved", "peak", "unit", "frac")}
    roofline.update({
        "kernel": dk["kernel"],
        "traffic": measured_traffic(path_name, wl.name, dk["kernel"]),
        "avg_launch_us": round(avg_t * 1e3, 3),
        "median_launch_us": dk["median_us"],
        "timed_by": "bracket of the K steps" if nl == 1 else "events around each launch",
        "work_per_launch": {"bytes": dk["bytes"], "flops": dk["flops"]},
        "launches_timed": args.steps if nl == 1 else nprof,
    })
    alg_bytes = wl.algorithmic_bytes()
    alg_flops = wl.algorithmic_flops()
    # the whole call over the step bracket (no events between its launches)
    whole = roofline_entry(alg_bytes, alg_flops, ms)
    whole.update({"call_us": round(ms * 1e3, 3),
                  "median_profiled_call_us": round(prof_call * 1e3, 3),
                  "algorithmic_bytes_per_call": alg_bytes,
                  "algorithmic_flops_per_call": alg_flops,
                  "traffic": measured_traffic(path_name, wl.name, None)})

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == 1 else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, row-softmax W; stand-in for the pages' image and "
                "video workloads)",
        "config": {
            "workload": "%s: B%d H%d N%d (%s grid, %s blocks, M=%d) d%d phi=%s%s%s" % (
                wl.name, wl.B, wl.H, wl.N, "x".join(map(str, wl.grid)),
                "x".join(map(str, wl.block)), wl.M, wl.d, "relu" if wl.phi == 0 else "elu+1",
                " causal" if wl.causal else "", "" if wl.norm else " no-norm"),
            "path": path_name,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "call_roofline": whole,
        "kernels": kernels,
        "timing": {
            "bracket_ms_per_step": round(ms, 6),
            "median_profiled_call_ms": round(prof_call, 6),
            "host_enqueue_us_per_call": round(host_s / args.steps * 1e6, 2),
            "host_calls_per_s": round(args.steps / host_s, 1),
            "launch_overhead_frac": round(max(0.0, (ms - prof_call) / ms), 4),
        },
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(inp, out, args.cpu_seconds)
        if not args.no_single_core:
            result["cpu_baseline_single_core"] = single_core_baselines(
                [n for n in ("tiny", "deit_t", "dit_xl2", "hires") if n != wl.name])

    print(json.dumps(result), flush=True)
    return 0


def roofline_of_call(gbs, tfs, alg_bytes, alg_flops):
    """Roofline object of a whole call timed by events (several kernels): the
    binding roofline is the larger of the HBM and bf16 MFMA fractions."""
    hbm, mfma = gbs / HBM_PEAK_GBS, tfs / BF16_PEAK_TFLOPS
    if hbm >= mfma:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s"}
    r.update({"frac": round(max(hbm, mfma), 4), "traffic": None, "hbm_frac": round(hbm, 4),
              "mfma_frac": round(mfma, 4), "algorithmic_bytes_per_launch": alg_bytes,
              "algorithmic_flops_per_launch": alg_flops})
    return r


def backward_bench(args):
    """One step = one mhla_backward call (recompute of the forward state, then
    dQ, dK, dV, dW) on the workload's inputs and a seeded upstream gradient."""
    import torch
    import token_level_head_mhla_amd as m
    from mhla_inputs import WORKLOADS, make_inputs, make_upstream_grad

    wl = WORKLOADS[args.workload]
    inp = make_inputs(wl)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, dy = dev(inp.q), dev(inp.k), dev(inp.v), dev(make_upstream_grad(wl))
    w = torch.from_numpy(inp.w).cuda()
    dq, dk, dv, dw = (torch.empty_like(x) for x in (q, k, v, w))
    shape = (wl.grid, wl.block)
    stream = torch.cuda.current_stream()

    def step():
        m.mhla_backward(q, k, v, w, dy, dq, dk, dv, dw, shape, wl.phi, wl.flags, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    t = wl.B * wl.H * wl.N * wl.d * 2
    alg_bytes = 7 * t + 2 * wl.H * wl.M * wl.M * 4   # read Q,K,V,dY,W; write dQ,dK,dV,dW
    d2 = wl.d * wl.d
    alg_flops = wl.B * wl.H * (12 * wl.N * d2 + 6 * wl.M * wl.M * d2)
    gbs = alg_bytes / (ms / 1e3) / 1e9
    tfs = alg_flops / (ms / 1e3) / 1e12
    roofline = roofline_of_call(gbs, tfs, alg_bytes, alg_flops)
    # counter-measured HBM bytes per call (blocked backward, committed summary)
    roofline["traffic"] = measured_traffic("backward", wl.name, None)
    print(json.dumps({
        "metric": "MHLA bwd tokens/s per GPU", "value": round(wl.B * wl.N / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "dtype": "bf16",
        "config": {"workload": wl.name, "pass": "backward"},
        "roofline": roofline}), flush=True)
    return 0


def decode_bench(args):
    """One step = one mhla_decode_step call: one new token for each of the B*H
    slices.  The timed region streams the whole sequence (N steps) after a
    warm-up pass; tokens/s counts B tokens per step.  Also reported: the
    prefill of the whole sequence as a prompt, and the sequence streamed with
    mhla_decode_steps in calls of 16 tokens."""
    import torch
    import token_level_head_mhla_amd as m
    from mhla_inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    if wl.grid[0] != 1 or wl.grid[1] != 1:
        print("bench.py: --decode needs a 1-D chunked workload", file=sys.stderr)
        return 2
    inp = make_inputs(wl)

    def dev(x):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return t.permute(2, 0, 1, 3).contiguous()   # [N, B, H, d]: token t is one slice

    qt, kt, vt = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    y = torch.empty_like(qt)
    nb, M = wl.block[2], wl.M
    state = torch.empty(m.mhla_decode_state_bytes(wl.B, wl.H, wl.d, M) // 4, dtype=torch.float32,
                        device="cuda")
    stream = torch.cuda.current_stream()

    def run_sequence():
        for t in range(wl.N):
            m.mhla_decode_step(qt[t], kt[t], vt[t], w, y[t], state, M, nb, t, wl.phi, wl.flags,
                               stream=stream)

    run_sequence()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    run_sequence()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / wl.N
    # prefill: the decode state from the whole sequence as a prompt, in one call
    kp = torch.from_numpy(np.ascontiguousarray(inp.k).view(np.int16)).view(torch.bfloat16).cuda()
    vp = torch.from_numpy(np.ascontiguousarray(inp.v).view(np.int16)).view(torch.bfloat16).cuda()

    def prefill():
        m.mhla_decode_prefill(kp, vp, w, state, M, nb, wl.phi, wl.flags, stream=stream)

    for _ in range(3):
        prefill()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(20):
        prefill()
    end.record(stream)
    torch.cuda.synchronize()
    prefill_ms = start.elapsed_time(end) / 20
    # several tokens per call: the sequence in calls of 16 tokens, inputs cut beforehand
    GROUP = 16
    qg, kg, vg = ([x[t:t + GROUP].permute(1, 2, 0, 3).contiguous()
                   for t in range(0, wl.N, GROUP)] for x in (qt, kt, vt))
    yg = [torch.empty_like(x) for x in qg]

    def run_groups():
        for c in range(len(qg)):
            m.mhla_decode_steps(qg[c], kg[c], vg[c], w, yg[c], state, M, nb, c * GROUP, wl.phi,
                                wl.flags, stream=stream)

    run_groups()
    torch.cuda.synchronize()
    start.record(stream)
    run_groups()
    end.record(stream)
    torch.cuda.synchronize()
    group_ms = start.elapsed_time(end) / wl.N
    E = wl.d * (wl.d + 1) * 4
    # per step and slice: prefix read, running summary read and written, q/k/v/y
    step_bytes = wl.B * wl.H * (3 * E + 4 * wl.d * 2)
    print(json.dumps({
        "metric": "MHLA incremental decode tokens/s per GPU",
        "value": round(wl.B / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": wl.N, "warmup": wl.N, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "dtype": "bf16 in, fp32 state",
        "config": {"workload": wl.name, "pass": "decode", "sequences": wl.B, "heads": wl.H},
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (ms / 1e3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "state_bytes_per_step": step_bytes},
        "prefill": {"prompt_tokens": wl.N, "us_per_call": round(prefill_ms * 1e3, 2),
                    "tokens_per_s": round(wl.B * wl.N / (prefill_ms / 1e3), 1)},
        "steps_per_call": {"tokens_per_call": GROUP, "us_per_token": round(group_ms * 1e3, 3),
                           "tokens_per_s": round(wl.B / (group_ms / 1e3), 1)}}),
          flush=True)
    return 0


# Sources of each path's kernels: a committed byte count applies only while
# these files are unchanged.
PATH_SOURCES = {
    "fused": ["k_fused.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
    "columns": ["k_cols.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
    "pairs": ["k_pairs.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
    "blocked": ["k_blocked.hpp", "k_causal.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
    # the blocked backward (mhla_backward with blocks of more than 16 tokens)
    "backward": ["k_backward.hpp", "k_blocked.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
}


def sources_digest(path_name):
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in PATH_SOURCES[path_name]:
        with open(os.path.join(root, "token_level_head_mhla_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path_name, workload, kernel):
    """HBM bytes per launch of `kernel` (per call when kernel is None) from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary of this path and
    workload, or None when there is none or the path's sources changed since
    it was taken."""
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(root, "profiles", "%s_%s_hbm_bytes.md" % (path_name, workload))
    if path_name not in PATH_SOURCES or not os.path.exists(summary):
        return None
    text = open(summary).read()
    digest = re.search(r"source_sha256_16: ([0-9a-f]{16})", text)
    if not digest or digest.group(1) != sources_digest(path_name):
        return None
    if kernel is None:
        key = "traffic_bytes_per_call"
    else:
        key = "traffic_bytes_per_launch\\[%s\\]" % kernel
    nbytes = re.search(key + r": (\d+)", text)
    return int(nbytes.group(1)) if nbytes else None


def _slice_inputs(inp, s0, s1):
    """fp64 Q, K, V of slices [s0, s1) (flattened over batch and head) as
    [1, s1-s0, N, d], and the matching per-slice W."""
    wl = inp.wl
    S = wl.B * wl.H
    flat = lambda x: x.reshape(S, wl.N, wl.d)[s0:s1][None]
    q, k, v = (inp.as_f64(flat(x)) for x in (inp.q, inp.k, inp.v))
    w = inp.w_f64[np.arange(s0, s1) % wl.H]
    return q, k, v, w


def time_oracle(inp, target_s, nthreads):
    """Times the fp64 blockwise oracle on a bounded sample of whole slices of
    the workload (repeated when one pass is short).  Returns (tokens/s,
    threads used, slices, runs, seconds, the sample's output)."""
    import oracle
    wl = inp.wl
    S = wl.B * wl.H
    q, k, v, w = _slice_inputs(inp, 0, 1)
    t0 = time.perf_counter()
    oracle.blockwise(q, k, v, w, wl.grid, wl.block, wl.phi, nthreads=nthreads, norm=wl.norm,
                     causal=wl.causal)
    per_slice = max(time.perf_counter() - t0, 1e-6)
    threads = oracle.threads() if nthreads <= 0 else nthreads
    ns = max(1, min(S, int(target_s * threads / per_slice)))
    if threads > 1:
        ns = min(S, max(ns, threads) // threads * threads)  # whole rounds of the thread pool
    q, k, v, w = _slice_inputs(inp, 0, ns)
    reps, elapsed, ref = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        ref = oracle.blockwise(q, k, v, w, wl.grid, wl.block, wl.phi, nthreads=nthreads,
                               norm=wl.norm, causal=wl.causal)
        elapsed += time.perf_counter() - t0
        reps += 1
        if elapsed >= 0.8 * target_s or reps >= 2000:
            break
    return reps * ns * wl.N / elapsed, threads, ns, reps, elapsed, ref


def cpu_baseline(inp, out_dev, target_s):
    """The fp64 oracle (blockwise C, OpenMP over slices, all host threads)
    timed on this host on a bounded sample of whole slices of the same
    workload; also reports the GPU output's error on that sample."""
    wl = inp.wl
    S = wl.B * wl.H
    rate, threads, ns, reps, elapsed, ref = time_oracle(inp, target_s, 0)
    y = out_dev.reshape(S, wl.N, wl.d)[:ns].float().cpu().numpy().astype(np.float64)
    ref = ref.reshape(ns, -1)
    num = np.abs(y.reshape(ns, -1) - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    err = float((num / np.where(den == 0, 1, den)).max())
    base = {
        "value": round(rate, 1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "fp64 blockwise oracle on %d of the %d (batch, head) slices (%d tokens each), "
                  "%d run(s), %.1f s wall, %d threads" % (ns, S, wl.N, reps, elapsed, threads),
    }
    parity = {"max_slice_rel_err": err, "slices_checked": ns,
              "gate": 1e-5 if wl.dtype == 0 else 1e-2}
    return base, parity


def single_core_baselines(names, target_s=2.5):
    """The same oracle on one thread, on bounded samples of the smaller
    workloads (their throughput per core)."""
    from mhla_inputs import WORKLOADS, make_inputs
    res = []
    for name in names:
        inp = make_inputs(WORKLOADS[name])
        rate, threads, ns, reps, elapsed, _ = time_oracle(inp, target_s, 1)
        res.append({"workload": name, "value": round(rate, 1), "unit": "tokens/s", "cores": 1,
                    "kind": "oracle", "sample": "%d of %d slices, %d run(s), %.2f s" % (
                        ns, inp.wl.B * inp.wl.H, reps, elapsed)})
    return res


if __name__ == "__main__":
    sys.exit(main())
