#!/usr/bin/env python3
"""Benchmark of the MHLA forward on one MI355X.

One step = one mhla_forward call: the whole hot path (block summaries,
multi-head mixing, readout) over one batch of seeded synthetic input that is
already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload deit_t] [--path auto]

The default workload is the DeiT-T-shaped bf16 case (B64 H3 N196 as a 14x14
grid of 7x7 blocks, so M=4; d64; elu+1).  The other workloads (tiny,
dit_xl2, hires, video) can be selected for study.

  python bench.py --copy-mb 256

times a plain device copy of that size instead (the reference kernel for
scaling the HBM byte counters of a profiler run).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
METRIC = "MHLA fwd tokens/s per GPU and % of bf16 MFMA / HBM roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deit_t")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "generic", "fused", "pairs", "blocked", "columns"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="time a plain device copy of this many MB instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (mhla_backward) instead of the forward")
    ap.add_argument("--decode", action="store_true",
                    help="time token-by-token causal inference (mhla_decode_step) over the "
                         "workload's sequence instead (1-D chunked workloads, e.g. lm_causal)")
    return ap.parse_args()


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
    kernels = {1: ["k_summary_valu", "k_mix_valu", "k_readout_valu"], 2: ["k_fused"],
               3: ["k_pairs"], 4: ["k_summary_mfma", "k_mix_mfma", "k_readout_mfma"],
               5: ["k_cols"]}[path]
    if wl.causal:
        kernels = ["k_summary_mfma", "k_mix_mfma", "k_readout_causal"]

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

    def step():
        m.mhla_forward_ex(q, k, v, w, out, shape, wl.phi, wl.flags, path, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events recorded on the launch stream bracket exactly the K steps.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens = wl.B * wl.N
    value = tokens / (ms / 1e3)

    alg_bytes = wl.algorithmic_bytes()
    alg_flops = wl.algorithmic_flops()
    hbm_frac = alg_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    mfma_frac = alg_flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS
    bound = "hbm" if hbm_frac >= mfma_frac else "mfma"
    if bound == "hbm":
        achieved, peak, unit = alg_bytes / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = alg_flops / (ms / 1e3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    roofline = {
        "bound": bound,
        "kernel": kernels[0] if len(kernels) == 1 else "+".join(kernels),
        "achieved": round(achieved, 1),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(kernels[0], wl.name) if len(kernels) == 1 else None,
        "algorithmic_bytes_per_launch": alg_bytes,
        "algorithmic_flops_per_launch": alg_flops,
        "avg_launch_us": round(ms * 1e3, 3),
    }

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
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(inp, out, args.cpu_seconds)

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
    print(json.dumps({
        "metric": "MHLA bwd tokens/s per GPU", "value": round(wl.B * wl.N / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "dtype": "bf16",
        "config": {"workload": wl.name, "pass": "backward"},
        "roofline": roofline_of_call(gbs, tfs, alg_bytes, alg_flops)}), flush=True)
    return 0


def decode_bench(args):
    """One step = one mhla_decode_step call: one new token for each of the B*H
    slices.  The timed region streams the whole sequence (N steps) after a
    warm-up pass; tokens/s counts B tokens per step."""
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
                     "traffic": None, "state_bytes_per_step": step_bytes}}),
          flush=True)
    return 0


# Sources that define each roofline kernel; a committed byte count applies only
# while these files are unchanged.
KERNEL_SOURCES = {"k_fused": ["k_fused.hpp", "mhla_mfma.hpp", "mhla_common.hpp"],
                  "k_cols": ["k_cols.hpp", "mhla_mfma.hpp", "mhla_common.hpp"]}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary for this kernel and workload, or None when there is none or the
    kernel's sources changed since it was taken."""
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(root, "profiles", "%s_%s_hbm_bytes.md" % (kernel, workload))
    if kernel not in KERNEL_SOURCES or not os.path.exists(summary):
        return None
    text = open(summary).read()
    nbytes = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    digest = re.search(r"source_sha256_16: ([0-9a-f]{16})", text)
    if not nbytes or not digest:
        return None
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(root, "token_level_head_mhla_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return int(nbytes.group(1)) if h.hexdigest()[:16] == digest.group(1) else None


def cpu_baseline(inp, out_dev, target_s):
    """The fp64 oracle (blockwise C, OpenMP over slices) timed on this host on
    a bounded sample of the same workload; also reports the GPU output's error
    on that sample."""
    import oracle
    wl = inp.wl
    q, k, v, w = inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64
    threads = oracle.threads()
    # size the sample (whole batch items, all heads) for about target_s seconds
    t0 = time.perf_counter()
    oracle.blockwise(q[:1, :1], k[:1, :1], v[:1, :1], w[:1], wl.grid, wl.block, wl.phi,
                     norm=wl.norm, causal=wl.causal)
    per_slice = max(time.perf_counter() - t0, 1e-6)
    n_b = max(1, min(wl.B, int(target_s * threads / per_slice / wl.H)))
    reps, elapsed, ref = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        ref = oracle.blockwise(q[:n_b], k[:n_b], v[:n_b], w, wl.grid, wl.block, wl.phi,
                               norm=wl.norm, causal=wl.causal)
        elapsed += time.perf_counter() - t0
        reps += 1
        if elapsed >= 0.8 * target_s or reps >= 2000:
            break
    tokens = reps * n_b * wl.N
    y = out_dev[:n_b].float().cpu().numpy().astype(np.float64)
    num = np.abs(y - ref).reshape(n_b * wl.H, -1).max(axis=1)
    den = np.abs(ref).reshape(n_b * wl.H, -1).max(axis=1)
    err = float((num / np.where(den == 0, 1, den)).max())
    base = {
        "value": round(tokens / elapsed, 1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "fp64 blockwise oracle on batch items 0..%d of %d (all %d heads), %d run(s), "
                  "%.1f s wall" % (n_b - 1, wl.B, wl.H, reps, elapsed),
    }
    parity = {"max_slice_rel_err": err, "slices_checked": n_b * wl.H,
              "gate": 1e-5 if wl.dtype == 0 else 1e-2}
    return base, parity


if __name__ == "__main__":
    sys.exit(main())
