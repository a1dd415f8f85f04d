#!/usr/bin/env python3
"""Benchmark of the MHLA forward on one MI355X.

One step = one mhla_forward call (the whole hot path: block summaries,
multi-head mixing and readout) over one batch of seeded synthetic input that
is already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload deit_t] [--path auto]

The default workload is the DeiT-T-shaped bf16 case (B64 H3 N196 as a 14x14
grid, 7x7 blocks so M=4, d64, elu+1).  Other workloads (tiny, dit_xl2, hires,
video) can be selected for study; they are parity-test cases, not the
reported line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deit_t")
    ap.add_argument("--path", default="auto", choices=["auto", "generic", "fused", "pairs", "blocked"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the (batch, head) slices shard across GPUs with no communication, but that "
              "launcher is not part of this build)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import token_level_head_mhla_amd as m
    from mhla_inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    path = {"auto": m.MHLA_PATH_AUTO, "generic": m.MHLA_PATH_GENERIC,
            "fused": m.MHLA_PATH_FUSED, "pairs": m.MHLA_PATH_PAIRS,
            "blocked": m.MHLA_PATH_BLOCKED}[args.path]
    shape = (wl.grid, wl.block)
    if path == m.MHLA_PATH_AUTO:
        path = m.mhla_plan(wl.B, wl.H, wl.N, wl.d, m.BlockShape.make(*shape), wl.phi, wl.dtype)
    path_name = {1: "generic", 2: "fused", 3: "pairs", 4: "blocked"}[path]
    n_kernels = {1: 3, 2: 1, 3: 1, 4: 3}[path]

    inp = make_inputs(wl)

    def dev(x):
        if wl.dtype == 1:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w = torch.from_numpy(inp.w).cuda()
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    def step():
        m.mhla_forward_path(q, k, v, w, out, shape, wl.phi, path)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    tokens = wl.B * wl.N
    value = tokens / (ms / 1e3)

    alg_bytes = wl.algorithmic_bytes()
    achieved = alg_bytes / (ms / 1e3) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "k_fused (whole forward)" if n_kernels == 1 else
                  "whole step (%d kernels: summary, mixing, readout)" % n_kernels,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": None,
        "algorithmic_bytes_per_launch": alg_bytes,
        "avg_launch_us": round(ms * 1e3, 3),
    }

    result = {
        "metric": "MHLA fwd tokens/s per GPU and % of bf16 MFMA / HBM roofline",
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
        "data": "synthetic (seeded N(0,1) Q/K/V, row-softmax W)",
        "config": {
            "workload": "%s: B%d H%d N%d (%s grid, %s blocks, M=%d) d%d phi=%s" % (
                wl.name, wl.B, wl.H, wl.N, "x".join(map(str, wl.grid)),
                "x".join(map(str, wl.block)), wl.M, wl.d, "relu" if wl.phi == 0 else "elu+1"),
            "path": path_name,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(inp, out, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(inp, out_dev, target_s):
    """The fp64 oracle (blockwise C, OpenMP) timed on this host on a bounded
    sample of the same workload; also reports the GPU output's error on it."""
    import oracle
    wl = inp.wl
    q, k, v, w = inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64
    # sample: whole slices, enough of them for about target_s of CPU time
    S = wl.B * wl.H
    t0 = time.perf_counter()
    oracle.blockwise(q[:1, :1], k[:1, :1], v[:1, :1], w[:1], wl.grid, wl.block, wl.phi)
    per_slice = max(time.perf_counter() - t0, 1e-6)
    threads = oracle.threads()
    n_b = max(1, min(wl.B, int(target_s * threads / per_slice / wl.H)))
    reps, elapsed, ref = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        ref = oracle.blockwise(q[:n_b], k[:n_b], v[:n_b], w, wl.grid, wl.block, wl.phi)
        elapsed += time.perf_counter() - t0
        reps += 1
        if elapsed >= target_s or reps >= 50:
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
        "sample": "first %d of %d batch items (all %d heads), %d run(s), %.1f s" % (
            n_b, wl.B, wl.H, reps, elapsed),
    }
    parity = {"max_slice_rel_err": err, "slices_checked": n_b * wl.H,
              "gate": 1e-5 if wl.dtype == 0 else 1e-2}
    return base, parity


if __name__ == "__main__":
    sys.exit(main())
