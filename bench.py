#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan (S6) forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long-context-128k]

A step is one ssm_scan_fwd call over the whole workload (every stage of the
hot path: step size, discretisation, chunk carries, carry fold, rescan with
readout, gate, store), inputs already resident in HBM.  Prints one JSON line.

Default workload: long-context-128k (batch 1, 131072 tokens, 2048 channels,
N = 16, bf16 io, fp32 state), the largest of the scan configurations that
fit one GPU, and the one that exercises the chunk carries and their combine.

Timing: the GPU's clocks ramp up over the first tens of milliseconds of
load, so the step is first run untimed until 250 ms have passed (reported
as clock_settle), then W untimed warm-up steps, then K steps bracketed by
synchronisations and HIP events on the stream the library launches on: that
region gives ms_per_step and value.  Events recorded between kernels slow a
step down (each one is a barrier on the queue), so the dominant kernel's own
duration is taken over another K steps in which the library brackets only
that kernel with events on its stream (ssm_timing_enable); the roofline uses
that average.  A third pass brackets every kernel for the per-kernel
breakdown.

Roofline.  The bound the pages name for this layer is HBM bandwidth, so
`roofline` holds the dominant kernel (s6_chunk_out, one full pass of the
method over every element per launch) against 8 TB/s: achieved = the
workload's algorithmic bytes (x, delta, z read and y written once, B and C
read once, parameters read, h_L written) / that kernel's average duration.
On MI355X the kernel is in fact limited by vector-ALU issue: every element
needs 16 exponentials and ~64 fp32 multiply/FMA operations for 8 bytes.
`valu` reports that separately, in issue slots (not flops): a full-rate slot
is one lane of a wave64 fp32 add/mul/FMA with VGPR operands, which gfx950
issues every 2 cycles per SIMD (32 lanes per cycle and SIMD; measured), so
256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 78.6e12 slots/s.  Transcendentals
(exp, log, rcp) count as four slots.  The method's work per (b, t, d)
element is 152 slots:
  16 states x (mul for Delta*A, exp = 4, mul for Delta*x*B, fma for h, fma for y) = 128
  softplus (exp 4 + log 4 + 3) = 11, Delta*x 1, skip 1, silu gate (exp 4 + rcp 4 + 3) = 11.
(an operand read from an SGPR halves an instruction's issue rate; that is
the kernel's cost, not the method's, and is not counted).

dtype is the arithmetic type of the path (fp32 state and arithmetic);
config.io is the storage type of x, delta, z, B, C and y.
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
PEAK_VALU_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12    # 157.3, fp32 vector (VGPR operands, no packed math)
PEAK_VALU_SLOTS = 256 * 4 * 32 * 2.4e9                 # 78.6e12 full-rate fp32 lane issue slots per second
DEFAULT_WORKLOAD = "long-context-128k"
SETTLE_MS = 250.0                   # untimed load before the warm-up steps, for the clocks to ramp up
CPU_POOL_MAX = 16                   # worker processes of the pooled CPU baseline (the host's CPU share)
SLOTS_PER_ELEMENT = 152
DOMINANT = "s6_chunk_out"          # the output pass: one full pass of the method per launch
# bench workload -> (what is timed, the named input workload it runs on)
WORKLOADS = {"mamba-130m-layer": ("scan", "mamba-130m-layer"), "mamba-2.8b-layer": ("scan", "mamba-2.8b-layer"),
             "long-context-128k": ("scan", "long-context-128k"), "decode-256x5120": ("decode", None),
             "mamba-130m-layer-bwd": ("bwd", "mamba-130m-layer"), "mamba-2.8b-layer-bwd": ("bwd", "mamba-2.8b-layer"),
             "mamba-130m-layer-conv": ("conv", "mamba-130m-layer"), "decode-256x5120-conv": ("decode", None),
             "mamba2-2.7b-layer": ("ssd", "mamba2-2.7b-layer"),
             "mamba2-2.7b-layer-n64": ("ssd", "mamba2-2.7b-layer-n64"),
             "mamba2-2.7b-layer-n256": ("ssd", "mamba2-2.7b-layer-n256"),
             "mamba2-long-context-128k": ("ssd", "mamba2-long-context-128k")}
PEAK_BF16_TFLOPS = 2500.0           # dense bf16 matrix-core peak
CONV_K = 4                          # width of the fused local convolution in the -conv workloads
CONV_SLOTS = 14                     # per element: 4 FMA + silu (exp 4, rcp 4, add, mul)
# Backward: algorithmic full-rate fp32 VALU slots per element (b, t, d), exp/log/rcp counted as 4:
#   state recompute: softplus 11 + Delta*x 1 + 16 x (mul, exp, mul, fma) 112          = 124
#   readout for the gate gradient: 16 FMA + skip                                       = 17
#   gate gradient (sigmoid: exp 4 + rcp 4, silu, derivative: 5)                        = 13
#   adjoint step: 16 x (mu, du, dC term, mul, exp, q, w, sum w A, dA, dB term)          = 208
#   per-token tail: sigmoid(v) from the softplus exponential (rcp 4), dx, dDelta,
#   ddelta, dD, dbias (8)                                                              = 12
#   channel sums of dB and dC: one add per value per channel                           = 32
BWD_SLOTS_PER_ELEMENT = 406
BWD_DOMINANT = "s6_chunk_bwd"
KERNEL_SOURCES = ["selective_state_space_39_amd/csrc/s6_kernels.hip",
                  "selective_state_space_39_amd/csrc/s6_device.h",
                  "selective_state_space_39_amd/csrc/s6_common.h"]
BWD_KERNEL_SOURCES = KERNEL_SOURCES + ["selective_state_space_39_amd/csrc/s6_bwd.hip"]
SSD_KERNEL_SOURCES = ["selective_state_space_39_amd/csrc/ssd_kernels.hip", "selective_state_space_39_amd/csrc/ssd_common.h",
                      "selective_state_space_39_amd/csrc/s6_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(batch, L, D, N=16, io_bytes=2):
    """x, delta, z read and y written once; B and C read once; A, Dskip, dt_bias read; h_L written."""
    return (4 * batch * L * D * io_bytes + 2 * batch * L * N * io_bytes + D * (N + 2) * 4 + batch * D * N * 4)


def kernel_source_hash(workload=""):
    """Hash of the sources the workload's kernels are compiled from."""
    h = hashlib.sha256()
    srcs = (BWD_KERNEL_SOURCES if workload.endswith("-bwd") else
            SSD_KERNEL_SOURCES if workload.startswith("mamba2") else KERNEL_SOURCES)
    for p in srcs:
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
    if not rec or rec.get("source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


CALIB_BYTES = 256 << 20           # copy-kernel calibration size
CALIB_REPS = 3


def copy_calibration():
    """A plain device-to-device copy of known size, for FETCH_SIZE / WRITE_SIZE calibration."""
    import torch
    a = torch.ones(CALIB_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(CALIB_REPS):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": CALIB_BYTES, "reps": CALIB_REPS}))


def _pmc(path, counter, kname):
    import csv
    import re
    pat = re.compile(r"(^|[^A-Za-z0-9_])" + re.escape(kname) + r"($|[^A-Za-z0-9_])")
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"])]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kname!r} in {path}")
    return sum(vals) / len(vals)


def record_traffic(workload, fetch_csv, write_csv, calib_fetch_csv, calib_write_csv):
    """HBM bytes per launch of each library kernel from rocprofv3 --pmc runs (KiB per dispatch),
    each counter scaled by what it reads for the copy kernel of known size."""
    f_cal = CALIB_BYTES / 1024 / _pmc(calib_fetch_csv, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    w_cal = CALIB_BYTES / 1024 / _pmc(calib_write_csv, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    rec = {}
    for kname in ("s6_chunk_out", "s6_chunk_carry", "s6_carry_scan", "s6_step", "s6_bwd_carries",
                  "s6_carry_scan2", "s6_chunk_bwd", "s6_bwd_reduce", "ssd_gram", "ssd_chunked", "ssd_seg_local",
                  "ssd_seg_fold"):
        try:
            fk, wk = _pmc(fetch_csv, "FETCH_SIZE", kname), _pmc(write_csv, "WRITE_SIZE", kname)
        except SystemExit:
            continue
        rec[kname] = {"bytes_per_launch": round((fk * f_cal + wk * w_cal) * 1024),
                      "fetch_kib_raw": fk, "write_kib_raw": wk, "source_hash": kernel_source_hash(workload)}
    t[workload] = rec
    t["_calibration"] = {"fetch_factor": round(f_cal, 4), "write_factor": round(w_cal, 4),
                         "copy_bytes": CALIB_BYTES}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
    print(json.dumps(t[workload]))


FLUSH_BYTES = 1 << 30          # four times the 256 MB Infinity Cache (MALL)


def flushed_timing(step, stream, algorithmic_bytes, elements, reps=30):
    """Single steps with the MALL (and L2) flushed by an untimed 1 GiB device write before each one:
    median, p10 and p90 over `reps` repetitions (events on the step's stream), and the HBM fraction of
    the algorithmic bytes at the median.  This is the pure-HBM figure; `value` above is the hot loop."""
    import torch
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=stream.device)
    ev = []
    torch.cuda.synchronize()
    for i in range(reps):
        buf.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: ms[min(len(ms) - 1, int(round(f * (len(ms) - 1))))]
    med = q(0.5)
    gbps = algorithmic_bytes / (med * 1e-3) / 1e9
    del buf
    return {"reps": reps, "flush_bytes": FLUSH_BYTES, "median_ms": round(med, 5), "p10_ms": round(q(0.1), 5),
            "p90_ms": round(q(0.9), 5), "elements_per_s": round(elements / (med * 1e-3), 1),
            "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4)}


_POOL_WORK = {}


def _pool_strip(i):
    """One channel strip of the scan workload set up in _POOL_WORK (inherited through fork)."""
    import oracle
    s, cs = _POOL_WORK["s"], _POOL_WORK["cs"]
    g = slice(cs * i, cs * (i + 1))
    oracle.scan_fwd(s.x[..., g], s.delta[..., g], s.A[g], s.B, s.C, s.Dskip[g], s.dt_bias[g], z=s.z[..., g], io=s.io)
    return os.getpid()


def cpu_baseline_strips(s, cs=128, min_seconds=10.0):
    """The float64 oracle as it stands, on the host, over channel strips of the workload (every token).

    single core: strips run one after another until min_seconds have passed;
    pool: every strip of the workload at once over a pool of forked worker processes
    (min(host CPUs, 16) of them), i.e. the whole workload, timed wall-clock.
    Must run before the process touches the GPU (the workers are forked from it)."""
    import multiprocessing as mp
    b, L, D, _ = s.shape
    strips = max(1, D // cs)
    _POOL_WORK.update(s=s, cs=cs)
    calls, elapsed = 0, 0.0
    while calls < strips and (calls == 0 or elapsed < min_seconds):
        t0 = time.perf_counter()
        _pool_strip(calls)
        elapsed += time.perf_counter() - t0
        calls += 1
    single = calls * b * L * cs / elapsed
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:
        host = os.cpu_count() or 1
    workers = max(1, min(host, CPU_POOL_MAX, strips))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        t0 = time.perf_counter()
        pids = pool.map(_pool_strip, range(strips), chunksize=1)
        wall = time.perf_counter() - t0
    _POOL_WORK.clear()
    pooled = strips * b * L * cs / wall
    return {"value": round(pooled, 1), "unit": "elements/s", "cores": len(set(pids)), "kind": "oracle",
            "sample": f"the whole workload as {strips} strips of {cs} channels ({b}x{L}x{cs}, every token) over a "
                      f"pool of {workers} forked processes, {wall:.1f} s wall; NumPy float64, one thread per process "
                      f"(host shows {host} CPUs)",
            "single_core": {"value": round(single, 1), "unit": "elements/s", "cores": 1,
                            "sample": f"{calls} strip(s) of {cs} channels one after another, {elapsed:.1f} s"}}


def settle(step, min_ms=None):
    """Run the step untimed until min_ms of wall time have passed (the clocks ramp up under load)."""
    import torch
    if min_ms is None:
        min_ms = SETTLE_MS
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
    return {"steps": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def cpu_sampled(call, elements_per_call, what, min_seconds=10.0, max_calls=400):
    """The float64 oracle as it stands, on the host: call(i) runs the i-th piece
    of the workload (a strip of channels or heads, or one decode step) and is
    repeated until min_seconds have passed; the rate is elements per second."""
    calls, elapsed = 0, 0.0
    while calls < max_calls and (calls == 0 or elapsed < min_seconds):
        t0 = time.perf_counter()
        call(calls)
        elapsed += time.perf_counter() - t0
        calls += 1
    return {"value": calls * elements_per_call / elapsed, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} x {what}, {elapsed:.1f} s; NumPy float64, single-threaded"}


def decode_bytes(batch, D, N=16, io_bytes=2):
    """State read and written; x, delta, z read and y written; B, C read; A, Dskip, dt_bias read."""
    return batch * D * (2 * N * 4 + 4 * io_bytes) + 2 * batch * N * io_bytes + D * (N + 2) * 4


def bench_decode(args):
    """Chained single-token decode steps against the cached fp32 state (256 x 5120 x 16).

    Eight pre-generated tokens are cycled so inputs stay resident in HBM.  The
    84 MB state is read and written every step; between steps it may stay in
    the 256 MB Infinity Cache, as it would in a serving loop.  This path is
    HBM-bound: the roofline is bytes against 8 TB/s.
    """
    import torch
    from selective_state_space_39_amd import binding, inputs
    batch, D = 256, 5120
    dev = torch.device("cuda:0")
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    f32 = lambda a: torch.from_numpy(a).to(dev)
    bf = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    toks = [inputs.decode_token(i, batch, D) for i in range(8)]
    dtoks = [tuple(bf(getattr(t, n)) for n in ("x", "delta", "z", "B", "C")) for t in toks]
    tA, tD, tb = f32(A), f32(Dskip), f32(dt_bias)
    h = f32(h0)
    y = torch.empty((batch, D), dtype=torch.bfloat16, device=dev)
    it = [0]

    conv = args.workload.endswith("-conv")
    if conv:
        cp = inputs.make_conv_params(batch, D, CONV_K, io="bf16", seed=inputs.DECODE_WORKLOAD["seed"], with_init=True)
        cw, cb = f32(cp.w), f32(cp.b)
        cstate = bf(cp.init)

    def step():
        x, dl, z, B, C = dtoks[it[0] & 7]
        it[0] += 1
        if conv:
            binding.conv_state_update(h, cstate, x, cw, cb, dl, tA, B, C, tD, tb, z=z, out=y)
        else:
            binding.state_update(h, x, dl, tA, B, C, tD, tb, z=z, out=y)

    settled = settle(step)
    for _ in range(args.warmup):
        step()
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

    ms_per_step = timed(args.steps) / args.steps
    # a step is one s6_step launch and the launches run back to back, so the
    # timed region's average is the kernel's own duration; the library's event
    # pair around each launch adds a few microseconds of dispatch to a kernel
    # this short and is reported beside it
    avg_ms = ms_per_step
    binding.timing_collect()
    binding.timing_enable(True, "s6_step")
    timed(args.steps)
    binding.timing_enable(False)
    c, kms = binding.timing_collect()["s6_step"]
    pair_ms = kms / c
    abytes = decode_bytes(batch, D) + (2 * batch * (CONV_K - 1) * D * 2 + D * (CONV_K + 1) * 4 if conv else 0)
    achieved = abytes / (avg_ms * 1e-3) / 1e9
    out = {"metric": METRIC, "value": round(batch * D / (ms_per_step * 1e-3), 1), "unit": "elements/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "clock_settle": settled,
           "config": {"workload": f"{args.workload} {'ssm_conv_state_update' if conv else 'ssm_state_update'}",
                      "batch": batch, "D": D, "N": 16, "io": "bf16", "state": "f32", "gated": True,
                      **({"conv_k": CONV_K} if conv else {})},
           "hbm": {"achieved_gbps": round(abytes / (ms_per_step * 1e-3) / 1e9, 1), "peak_gbps": PEAK_HBM_GBPS,
                   "frac": round(abytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                   "algorithmic_bytes_per_step": abytes},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM_GBPS, 4),
                        "traffic": measured_traffic(args.workload, "s6_step"), "kernel": "s6_step",
                        "avg_launch_ms": round(avg_ms, 5), "event_pair_ms": round(pair_ms, 5),
                        "work": f"{abytes} algorithmic bytes per launch (136 B per (b, d) + B/C + parameters"
                                + (", + the conv state read and written" if conv else "") + ")"},
           "mall_flushed": None if args.no_flushed else flushed_timing(step, stream, abytes, batch * D)}
    if not args.no_cpu_baseline:
        import oracle
        st = {"h": h0.astype("float64"), "conv": cp.init if conv else None}

        def one(i):
            t = toks[i & 7]
            if conv:
                _, st["h"], st["conv"] = oracle.conv_state_update(st["conv"], st["h"], t.x, cp.w, cp.b, t.delta, A,
                                                                  t.B, t.C, Dskip, dt_bias, z=t.z, io="bf16")
            else:
                _, st["h"] = oracle.state_update(st["h"], t.x, t.delta, A, t.B, t.C, Dskip, dt_bias, z=t.z, io="bf16")
        out["cpu_baseline"] = cpu_sampled(one, batch * D, f"chained decode steps of the whole {batch}x{D} state")
    print(json.dumps(out), flush=True)


def bwd_algorithmic_bytes(batch, L, D, N=16, io_bytes=2):
    """x, delta, z, dout read and dx, ddelta, dz written once; B, C read; dB, dC (fp32) written;
    parameters read and their gradients written."""
    return (7 * batch * L * D * io_bytes + 2 * batch * L * N * (io_bytes + 4) + 2 * D * (N + 2) * 4)


def bench_bwd(args, name):
    """ssm_scan_bwd on a whole-sequence workload: gradients with respect to every input."""
    import torch
    from selective_state_space_39_amd import binding, inputs
    s = inputs.make_workload(name)
    batch, L, D, N = s.shape
    io = s.io
    go = inputs.make_grad_outputs(batch, L, D, N, io=io, seed=inputs.SCAN_WORKLOADS[name]["seed"],
                                  with_dh_last=False)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if io == "bf16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    f32 = lambda a: torch.from_numpy(a).to(dev)
    x, dl, z, B, C, dout = (to_dev(a) for a in (s.x, s.delta, s.z, s.B, s.C, go.dout))
    A, Dk, bias = f32(s.A), f32(s.Dskip), f32(s.dt_bias)
    io_code = binding.SSM_BF16 if io == "bf16" else binding.SSM_F32
    nws = binding.bwd_workspace_bytes(batch, L, D, io_code, args.chunk_len)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    chunk_len, n_chunks = binding.bwd_plan(batch, L, D, io_code, args.chunk_len)
    grads = binding.scan_bwd(x, dl, A, B, C, Dk, bias, dout, z=z, chunk_len=args.chunk_len, workspace=ws)

    def step():
        binding.scan_bwd(x, dl, A, B, C, Dk, bias, dout, z=z, chunk_len=args.chunk_len, workspace=ws, grads=grads)

    settled = settle(step)
    for _ in range(args.warmup):
        step()
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

    ms_per_step = timed(args.steps) / args.steps
    binding.timing_collect()
    binding.timing_enable(True, BWD_DOMINANT)
    timed(args.steps)
    binding.timing_enable(False)
    launches, kms = binding.timing_collect()[BWD_DOMINANT]
    avg_ms = kms / launches
    binding.timing_enable(True)
    ms_all = timed(args.steps) / args.steps
    binding.timing_enable(False)
    breakdown = binding.timing_collect()

    E = batch * L * D
    abytes = bwd_algorithmic_bytes(batch, L, D, N, 2 if io == "bf16" else 4)
    hbm_gbps = abytes / (ms_per_step * 1e-3) / 1e9
    achieved = E * BWD_SLOTS_PER_ELEMENT * 2 / (avg_ms * 1e-3) / 1e12
    kernels = {n: {"launches": c, "avg_ms": round(t / c, 5)} for n, (c, t) in breakdown.items()}
    kernels["_note"] = (f"every kernel bracketed by events in a separate pass: {ms_all:.4f} ms per step "
                        f"with the events, {ms_per_step:.4f} without")
    out = {"metric": "selective-scan backward elements/s (B·L·D), 1 MI355X", "value": round(E / (ms_per_step * 1e-3), 1),
           "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic", "clock_settle": settled,
           "config": {"workload": f"{args.workload} ssm_scan_bwd", "batch": batch, "L": L, "D": D, "N": N, "io": io,
                      "state": "f32", "gated": True, "chunk_len": chunk_len, "n_chunks": n_chunks},
           "hbm": {"achieved_gbps": round(hbm_gbps, 1), "peak_gbps": PEAK_HBM_GBPS,
                   "frac": round(hbm_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes_per_step": abytes},
           "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(PEAK_VALU_TFLOPS, 2),
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_VALU_TFLOPS, 4),
                        "traffic": measured_traffic(args.workload, BWD_DOMINANT), "kernel": BWD_DOMINANT,
                        "avg_launch_ms": round(avg_ms, 5),
                        "work": f"{BWD_SLOTS_PER_ELEMENT} full-rate fp32 VALU slots (= {2 * BWD_SLOTS_PER_ELEMENT} "
                                f"FMA-equivalent flops) per element x {E} elements per launch"},
           "kernels": kernels,
           "mall_flushed": None if args.no_flushed else flushed_timing(step, stream, abytes, E)}
    if not args.no_cpu_baseline:
        import oracle
        cs = 128

        def one(i):
            g = slice(cs * i % D, cs * i % D + cs)
            oracle.scan_bwd(s.x[..., g], s.delta[..., g], s.A[g], s.B, s.C, s.Dskip[g], s.dt_bias[g], go.dout[..., g],
                            z=s.z[..., g], io=io)
        out["cpu_baseline"] = cpu_sampled(one, batch * L * cs,
                                          f"{cs}-channel strips of the workload ({batch}x{L}x{cs}, all tokens)")
    print(json.dumps(out), flush=True)


def ssd_bytes(batch, L, H, P, N, gated=True):
    """x read, y written (and z read) once; delta, B, C read; parameters read (bf16 io)."""
    return (batch * L * H * P * 2 * (3 if gated else 2) + batch * L * H * 2 + 2 * batch * L * N * 2 + H * 12)


def ssd_flops(batch, L, H, P, N, Q=64):
    """Matrix-core work of ssd_chunked: per head and chunk the causal half of the masked Q x Q x P
    product, the state term Q x N x P and the state update P x Q x N (2 flops per MAC).  C B^T, once per
    (batch row, chunk), is ssd_gram's (2 Q Q N per chunk) and not counted here."""
    chunks = -(-L // Q)
    return batch * chunks * H * (Q * Q * P + 2 * Q * N * P + 2 * P * Q * N)


def bench_ssd(args, name):
    """The SSD (Mamba-2 style) layer on the 2.7B-layer shape: 8 x 2048 tokens, 80 heads of 64, N = 128
    (or 64, 256 for the -n64, -n256 workloads)."""
    import torch
    from selective_state_space_39_amd import binding, inputs
    w = inputs.SSD_WORKLOADS[name]
    if args.heads:
        w = dict(w, H=args.heads)
        name = f"{name} with {args.heads} heads"
    s = inputs.make_ssd_inputs(w["batch"], w["L"], w["H"], w["P"], w["N"], seed=w["seed"])
    batch, L, H, P, N = s.shape
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(a).to(dev)
    x, dl, z, B, C = (bf(a) for a in (s.x, s.delta, s.z, s.B, s.C))
    A, Dk, bias = f32(s.A), f32(s.Dskip), f32(s.dt_bias)
    y = torch.empty_like(x)
    ws = torch.empty(binding.ssd_workspace_bytes(batch, L, H, N, P), dtype=torch.uint8, device=dev)

    def step():
        binding.ssd_fwd(x, dl, A, B, C, Dk, bias, z=z, out=y, return_last_state=False, workspace=ws)

    settled = settle(step)
    for _ in range(args.warmup):
        step()
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

    ms_per_step = timed(args.steps) / args.steps
    binding.timing_collect()
    binding.timing_enable(True, "ssd_chunked")
    timed(args.steps)
    binding.timing_enable(False)
    c, kms = binding.timing_collect()["ssd_chunked"]
    avg_ms = kms / c
    binding.timing_enable(True)
    timed(args.steps)
    binding.timing_enable(False)
    breakdown = {k: {"launches": n, "avg_ms": round(t / n, 5)} for k, (n, t) in binding.timing_collect().items()}
    E = batch * L * H * P
    abytes = ssd_bytes(batch, L, H, P, N)
    flops = ssd_flops(batch, L, H, P, N)
    gbps = abytes / (avg_ms * 1e-3) / 1e9
    tflops = flops / (avg_ms * 1e-3) / 1e12
    out = {"metric": "SSD layer elements/s (B·L·H·P), 1 MI355X", "value": round(E / (ms_per_step * 1e-3), 1),
           "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic", "clock_settle": settled,
           "config": {"workload": f"{name} ssm_ssd_fwd", "batch": batch, "L": L, "H": H, "P": P, "N": N,
                      "io": "bf16", "state": "f32", "gated": True, "chunk": 64,
                      "segments": binding.ssd_plan(batch, L, H, N, P)[0]},
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None if args.heads else measured_traffic(args.workload, "ssd_chunked"),
                        "kernel": "ssd_chunked", "avg_launch_ms": round(avg_ms, 5),
                        "work": f"{abytes} algorithmic bytes per launch (x, z read, y written, delta, B, C)"},
           "mfma": {"achieved_tflops": round(tflops, 1), "peak_tflops": PEAK_BF16_TFLOPS,
                    "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "flops_per_launch": flops},
           "kernels": breakdown,
           "mall_flushed": None if args.no_flushed else flushed_timing(step, stream, abytes, E)}
    if not args.no_cpu_baseline:
        import oracle
        hs = 4

        def one(i):
            g = slice(hs * i % H, hs * i % H + hs)
            oracle.ssd_fwd(s.x[:, :, g], s.delta[:, :, g], s.A[g], s.B, s.C, s.Dskip[g], s.dt_bias[g], z=s.z[:, :, g],
                           io=s.io)
        out["cpu_baseline"] = cpu_sampled(one, batch * L * hs * P,
                                          f"{hs}-head strips of the workload ({batch}x{L}x{hs}x{P}, all tokens)")
    print(json.dumps(out), flush=True)


def main():
    global SETTLE_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The clocks are settled by SETTLE_MS of untimed load before the warm-up
    # steps (settle()), so a few warm-up steps suffice.
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--chunk-len", type=int, default=0)
    ap.add_argument("--heads", type=int, default=0,
                    help="SSD workloads: run the layer with this many heads instead (an occupancy sweep; the "
                         "line's config then names the changed shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed load before the warm-up steps (0 for counter runs under a profiler)")
    ap.add_argument("--no-flushed", action="store_true",
                    help="skip the cache-flushed single steps (kernel traces then cover the timed loops only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (profile it for counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv files into profiles/traffic.json")
    args = ap.parse_args()
    SETTLE_MS = args.settle_ms
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards over batch rows and channels with no communication, so N GPUs "
              "run N independent copies).", file=sys.stderr)
        sys.exit(2)

    kind, name = WORKLOADS[args.workload]
    conv = args.workload.endswith("-conv")
    from selective_state_space_39_amd import inputs
    s = cpu = None
    if kind in ("scan", "conv"):
        s = inputs.make_workload(name)
        # the pooled oracle forks worker processes: before anything touches the GPU
        if not args.no_cpu_baseline and not conv:
            cpu = cpu_baseline_strips(s)

    import torch
    from selective_state_space_39_amd import binding
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if kind == "ssd":
        return bench_ssd(args, name)
    if kind == "decode":
        return bench_decode(args)
    if kind == "bwd":
        return bench_bwd(args, name)
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

    if conv:
        cp = inputs.make_conv_params(batch, D, CONV_K, io=io, seed=inputs.SCAN_WORKLOADS[name]["seed"])
        cw, cb = f32(cp.w), f32(cp.b)

        def step():
            binding.conv_scan_fwd(x, cw, cb, dl, A, B, C, Dk, bias, z=z, chunk_len=args.chunk_len, out=y,
                                  workspace=ws)
    else:
        def step():
            binding.scan_fwd(x, dl, A, B, C, Dk, bias, z=z, chunk_len=args.chunk_len, out=y, workspace=ws)

    settled = settle(step)
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
    if conv:                                        # conv taps and bias read, conv_last not requested
        abytes += D * (CONV_K + 1) * 4
    hbm_gbps = abytes / (ms_per_step * 1e-3) / 1e9

    dominant = DOMINANT
    launches, kms = kern[dominant]
    avg_ms = kms / launches
    achieved = abytes / (avg_ms * 1e-3) / 1e9       # one launch = one full pass over every element
    slots = SLOTS_PER_ELEMENT + (CONV_SLOTS if conv else 0)
    slot_rate = E * slots / (avg_ms * 1e-3)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(args.workload, dominant),
                "kernel": dominant, "avg_launch_ms": round(avg_ms, 5),
                "work": f"{abytes} algorithmic bytes per launch = {abytes / E:.4f} B per element x {E} elements "
                        f"(x, delta, z read and y written once, B and C read, parameters read, h_L written); "
                        f"one launch is one full pass of the method"}
    valu = {"unit": "full-rate fp32 VALU lane issue slots per second", "slots_per_element": slots,
            "achieved": round(slot_rate / 1e12, 3), "peak": round(PEAK_VALU_SLOTS / 1e12, 3), "scale": 1e12,
            "frac": round(slot_rate / PEAK_VALU_SLOTS, 4), "kernel": dominant,
            "note": "the method's issue slots per element (exp, log, rcp = 4 slots) over the dominant kernel's "
                    "duration: the limit this kernel actually meets on gfx950" + (
                        " (incl. the width-4 convolution)" if conv else "")}
    kernels = {n: {"launches": c, "avg_ms": round(t / c, 5)} for n, (c, t) in breakdown.items()}
    kernels["_note"] = (f"every kernel bracketed by events in a separate pass: {ms_all:.4f} ms per step "
                        f"with the events, {ms_per_step:.4f} without")

    out = {"metric": METRIC, "value": round(value, 1), "unit": "elements/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": f"{args.workload} {'ssm_conv_scan_fwd' if conv else 'ssm_scan_fwd'}",
                      "batch": batch, "L": L, "D": D, "N": N, "io": io, "state": "f32", "gated": True,
                      "chunk_len": chunk_len, "n_chunks": n_chunks, **({"conv_k": CONV_K} if conv else {})},
           "clock_settle": settled,
           "hbm": {"achieved_gbps": round(hbm_gbps, 1), "peak_gbps": PEAK_HBM_GBPS,
                   "frac": round(hbm_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes_per_step": abytes,
                   "note": "whole step (every kernel of the call) against 8 TB/s"},
           "roofline": roofline, "valu": valu, "kernels": kernels,
           "mall_flushed": None if args.no_flushed else flushed_timing(step, stream, abytes, E)}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    elif not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_sampled(
            lambda i: oracle.conv_scan_fwd(s.x, cp.w, cp.b, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, z=s.z, io=io),
            E, f"full passes of the workload ({batch}x{L}x{D}, convolution included)")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
