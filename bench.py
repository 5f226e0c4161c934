#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan (S6) forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba-130m-layer]

A step is one ssm_scan_fwd call over the whole workload (every stage of the
hot path: step size, discretisation, chunk carries, carry fold, rescan with
readout, gate, store), inputs already resident in HBM.  Prints one JSON line.

Timing: W untimed warm-up steps, then K steps bracketed by synchronisations
and HIP events on the stream the library launches on: that region gives
ms_per_step and value.  Events recorded between kernels slow a step down
(each one is a barrier on the queue), so the dominant kernel's own duration
is taken over another K steps in which the library brackets only that kernel
with events on its stream (ssm_timing_enable); the roofline uses that
average.  A third pass brackets every kernel for the per-kernel breakdown.

Roofline.  On MI355X this path is bound by vector-ALU issue, not HBM: every
element needs 16 exponentials and ~64 fp32 multiply/FMA operations for 8 bytes
of HBM traffic.  The work unit is an fp32 VALU issue slot of one lane (a
full-rate instruction; transcendentals issue at half rate and count as two),
reported as FMA-equivalent flops (2 per slot) against the chip's fp32 vector
peak without packed math: 256 CUs x 64 lanes x 2 x 2.4 GHz = 78.64 TFLOP/s.
The algorithmic work per (b, t, d) element is 112 slots = 224 flops:
  16 states x (mul for Delta*A, exp = 2, mul for Delta*x*B, fma for h, fma for y) = 96
  softplus (exp 2 + log 2 + 3) = 7, Delta*x 1, skip 1, silu gate (exp 2 + rcp 2 + 3) = 7.
The achieved HBM rate (algorithmic bytes / step time) and its fraction of
8 TB/s are reported next to it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan elements/s (B·L·D) and achieved HBM GB/s vs peak, 1 MI355X"
PEAK_HBM_GBPS = 8000.0
PEAK_VALU_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12        # 78.64, fp32 vector without packed math
SLOTS_PER_ELEMENT = 112
DOMINANT = "s6_chunk_out"          # the output pass: one full pass of the method per launch
WORKLOADS = {"mamba-130m-layer": 2, "mamba-2.8b-layer": 3, "long-context-128k": 4}
KERNEL_SOURCES = ["selective_state_space_39_amd/csrc/s6_kernels.hip",
                  "selective_state_space_39_amd/csrc/s6_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(batch, L, D, N=16, io_bytes=2):
    """x, delta, z read and y written once; B and C read once; A, Dskip, dt_bias read; h_L written."""
    return (4 * batch * L * D * io_bytes + 2 * batch * L * N * io_bytes + D * (N + 2) * 4 + batch * D * N * 4)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(s, min_seconds=10.0, max_passes=3):
    """The float64 oracle as it stands, on the host, over whole passes of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    b, L, D, _ = s.shape
    passes, elapsed = 0, 0.0
    while passes < max_passes and (passes == 0 or elapsed < min_seconds):
        t0 = time.perf_counter()
        oracle.scan_fwd(s.x, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, z=s.z, io=s.io)
        elapsed += time.perf_counter() - t0
        passes += 1
    value = passes * b * L * D / elapsed
    return {"value": value, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full pass(es) of the workload ({b}x{L}x{D}), {elapsed:.1f} s; "
                      f"NumPy float64 elementwise loop, single-threaded (BLAS pool {blas_threads} unused)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba-130m-layer", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk-len", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards over batch rows and channels with no communication, so N GPUs "
              "run N independent copies).", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_39_amd import binding, inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    k = WORKLOADS[args.workload]
    s = inputs.make_config(k)
    batch, L, D, N = s.shape
    io = s.io
    dev = torch.device("cuda:0")

    def to_dev(a):
        if io == "bf16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    f32 = lambda a: torch.from_numpy(a).to(dev)
    x, dl, z, B, C = (to_dev(a) for a in (s.x, s.delta, s.z, s.B, s.C))
    A, Dk, bias = f32(s.A), f32(s.Dskip), f32(s.dt_bias)
    y = torch.empty_like(x)
    io_code = binding.SSM_BF16 if io == "bf16" else binding.SSM_F32
    nws = binding.workspace_bytes(batch, L, D, io_code, args.chunk_len)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    chunk_len, n_chunks = binding.plan(batch, L, D, io_code, args.chunk_len)

    def step():
        binding.scan_fwd(x, dl, A, B, C, Dk, bias, z=z, chunk_len=args.chunk_len, out=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def timed(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # (1) the measured region: K whole steps, no events between kernels
    ms_total = timed(args.steps)
    ms_per_step = ms_total / args.steps
    # (2) the dominant kernel alone, bracketed by HIP events on its own stream
    #     over another K steps (the library records them around that launch)
    binding.timing_collect()
    binding.timing_enable(True, DOMINANT)
    timed(args.steps)
    binding.timing_enable(False)
    kern = binding.timing_collect()
    # (3) every kernel bracketed (events between kernels slow the step: breakdown only)
    binding.timing_enable(True)
    ms_all = timed(args.steps) / args.steps
    binding.timing_enable(False)
    breakdown = binding.timing_collect()

    E = batch * L * D
    value = E / (ms_per_step * 1e-3)
    abytes = algorithmic_bytes(batch, L, D, N, 2 if io == "bf16" else 4)
    hbm_gbps = abytes / (ms_per_step * 1e-3) / 1e9

    dominant = DOMINANT
    launches, kms = kern[dominant]
    avg_ms = kms / launches
    work_flops = E * SLOTS_PER_ELEMENT * 2          # one full pass of the method per launch
    achieved = work_flops / (avg_ms * 1e-3) / 1e12
    traffic = measured_traffic(args.workload, dominant)
    roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(PEAK_VALU_TFLOPS, 2),
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_VALU_TFLOPS, 4), "traffic": traffic,
                "kernel": dominant, "avg_launch_ms": round(avg_ms, 5),
                "work": f"{SLOTS_PER_ELEMENT} fp32 VALU slots (= {2 * SLOTS_PER_ELEMENT} FMA-equivalent flops) "
                        f"per element x {E} elements per launch"}
    kernels = {n: {"launches": c, "avg_ms": round(t / c, 5)} for n, (c, t) in breakdown.items()}
    kernels["_note"] = (f"every kernel bracketed by events in a separate pass: {ms_all:.4f} ms per step "
                        f"with the events, {ms_per_step:.4f} without")

    out = {"metric": METRIC, "value": round(value, 1), "unit": "elements/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": f"{args.workload} ssm_scan_fwd", "batch": batch, "L": L, "D": D, "N": N,
                      "io": io, "state": "f32", "gated": True, "chunk_len": chunk_len, "n_chunks": n_chunks},
           "hbm": {"achieved_gbps": round(hbm_gbps, 1), "peak_gbps": PEAK_HBM_GBPS,
                   "frac": round(hbm_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes_per_step": abytes},
           "roofline": roofline, "kernels": kernels}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
