"""ssm_scan_fwd_noalloc, the entry point for callers that cannot allocate:
its chunk carries go to the library's fixed per-GPU scratch instead of a
caller workspace.  Checked through the C ABI against ssm_scan_fwd, the entry
point it is a variant of: bit for bit with the same chunk plan, on two calls
in a row with the second smaller (the scratch keeps the first call's
contents), within the parity bound where the scratch forces another plan,
and size errors before anything runs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import TOL, dev, f32dev, host64, log, oracle_scan, rel_err
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _dev_args(s, h0=None):
    io = s.io
    return (dev(s.x, io), dev(s.delta, io), f32dev(s.A), dev(s.B, io), dev(s.C, io), f32dev(s.Dskip),
            f32dev(s.dt_bias)), dict(z=dev(s.z, io), h0=f32dev(h0))


def _both(pos, kw, chunk_len, chunk_len_noalloc=None):
    """ssm_scan_fwd (caller workspace) and ssm_scan_fwd_noalloc (library scratch) on the same inputs."""
    y1, h1 = binding.scan_fwd(*pos, chunk_len=chunk_len, **kw)
    y2 = torch.full_like(y1, float("nan"))
    h2 = torch.full_like(h1, float("nan"))
    torch.cuda.synchronize()
    # torch's count of allocation requests: frees (the garbage collector may
    # release an earlier test's tensors at any time) do not move it
    def allocs():
        st = torch.cuda.memory_stats()
        for key in ("allocation.all.allocated", "allocated.all.allocated"):
            if key in st:
                return st[key]
        raise KeyError("torch.cuda.memory_stats() has no allocation-request count")
    before = allocs()
    binding.scan_fwd_noalloc(*pos, chunk_len=chunk_len if chunk_len_noalloc is None else chunk_len_noalloc,
                             out=y2, h_last_out=h2, **kw)
    assert allocs() == before                              # the binding allocated nothing either
    torch.cuda.synchronize()
    return y1, h1, y2, h2


def test_two_calls_bit_equal_to_the_workspace_entry_point():
    # first call: 64 chunks of 64 tokens, 13 MB of carries, bf16 with h0
    s = inputs.make_scan_inputs(2, 4096, 1536, io="bf16", seed=(39, 41), with_h0=True)
    log("noalloc call 1: 2 x 4096 x 1536 bf16, chunk_len 64")
    pos, kw = _dev_args(s, s.h0)
    y1, h1, y2, h2 = _both(pos, kw, 64)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    # second call, smaller: fp32 io, ragged last chunk; the scratch still holds call 1's carries
    t = inputs.make_scan_inputs(1, 1000, 640, io="f32", seed=(39, 42))
    log("noalloc call 2: 1 x 1000 x 640 f32, chunk_len 96")
    pos, kw = _dev_args(t)
    y1, h1, y2, h2 = _both(pos, kw, 96)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    ry, rh = oracle_scan(t)
    ey, _ = rel_err(host64(y2), ry)
    eh, _ = rel_err(host64(h2), rh)
    log(f"call 2 against the oracle: y {ey:.2e}, h {eh:.2e}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_plan_limited_by_the_scratch():
    """At 1 x 131072 x 2048 the workspace plan's carries (68 MiB) exceed the scratch, so the no-allocation
    call runs another chunk plan: same function, another rounding order."""
    blk = inputs.make_scan_inputs(1, 8192, 2048, io="bf16", seed=(39, 43))
    tile = lambda a: np.ascontiguousarray(np.tile(a, (1, 16, 1)))
    s = inputs.ScanInputs(**{**blk.__dict__, "x": tile(blk.x), "delta": tile(blk.delta), "z": tile(blk.z),
                             "B": tile(blk.B), "C": tile(blk.C)})
    assert binding.workspace_bytes(1, 131072, 2048, binding.SSM_BF16, 0) > SCRATCH_BYTES
    log("noalloc: 1 x 131072 x 2048 bf16, automatic plans")
    pos, kw = _dev_args(s)
    y1, h1, y2, h2 = _both(pos, kw, 0)
    a, b = host64(y1), host64(y2)
    ey = float(np.max(np.abs(a - b))) / float(np.max(np.abs(a)))
    eh = float((h1 - h2).abs().max() / h1.abs().max())
    log(f"noalloc vs workspace plan: y {ey:.2e}, h {eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= 1e-4


def test_sizes_beyond_the_scratch_are_refused():
    """An explicit chunk plan whose carries exceed the scratch: SSM_ERR_WORKSPACE, nothing runs."""
    batch, L, D = 1, 65536, 2048
    x = torch.zeros((batch, L, D), dtype=torch.bfloat16, device="cuda")
    BC = torch.zeros((batch, L, 16), dtype=torch.bfloat16, device="cuda")
    A = torch.full((D, 16), -1.0, device="cuda")
    Dk = torch.ones(D, device="cuda")
    y = torch.full_like(x, 7.0)
    with pytest.raises(binding.SSMError) as e:
        binding.scan_fwd_noalloc(x, x.clone(), A, BC, BC.clone(), Dk, Dk.clone(), chunk_len=64, out=y)
    assert e.value.status == -6 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())                               # output untouched


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_capture_replays_match_eager():
    """The call captured into a HIP graph, the use it exists for, and replayed
    three times, each time on new inputs copied into the captured buffers,
    with eager calls and host synchronisation between the replays: every
    replay bit-equal to the same call made eagerly on the same inputs."""
    batch, L, D = 2, 700, 160
    s = inputs.make_scan_inputs(batch, L, D, io="bf16", seed=(39, 9500), with_h0=True)
    pos, kw = _dev_args(s, s.h0)
    y = torch.empty_like(pos[0])
    h = torch.empty((batch, D, 16), dtype=torch.float32, device="cuda")

    def call():
        binding.scan_fwd_noalloc(*pos, chunk_len=64, out=y, h_last_out=h, **kw)

    g = _capture(call)
    for rep in range(3):
        s2 = inputs.make_scan_inputs(batch, L, D, io="bf16", seed=(39, 9501 + rep), with_h0=True)
        pos2, kw2 = _dev_args(s2, s2.h0)
        for a, b in zip(pos, pos2):
            a.copy_(b)
        kw["z"].copy_(kw2["z"])
        kw["h0"].copy_(kw2["h0"])
        g.replay()
        torch.cuda.synchronize()
        ye, he = binding.scan_fwd_noalloc(*pos, chunk_len=64, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {rep}: y differs from the eager call"
        assert torch.equal(h, he), f"replay {rep}: h_last differs from the eager call"
        log(f"noalloc graph replay {rep} on new inputs: bit-exact")
