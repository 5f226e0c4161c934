"""The library's calls captured into a HIP graph and replayed (needs an MI355X).

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a serving loop can capture a call, or several
chained decode steps, once and replay them.  Every replay is checked bit for
bit against the same calls made eagerly, with eager work and host
synchronisation between the replays.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, f32dev, log
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu


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


def test_graph_decode_chain_replays_match_eager():
    batch, D, steps = 32, 640, 4
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    toks = [inputs.decode_token(s, batch, D) for s in range(steps)]
    dtok = [tuple(dev(getattr(t, n), "bf16") for n in ("x", "delta", "z", "B", "C")) for t in toks]
    tA, tD, tb = f32dev(A), f32dev(Dskip), f32dev(dt_bias)
    h = f32dev(h0)
    ys = [torch.empty((batch, D), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    def chain(state, outs):
        for s, (x, dl, z, B, C) in enumerate(dtok):
            binding.state_update(state, x, dl, tA, B, C, tD, tb, z=z, out=outs[s])

    g = _capture(lambda: chain(h, ys))
    # the warm-up and the capture run advanced nothing: capture does not execute, the warm-up did once
    he = f32dev(h0)
    ye = [torch.empty_like(y) for y in ys]
    chain(he, ye)                              # the eager twin of the warm-up
    h.copy_(he)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        chain(he, ye)                          # eager, between replays
        torch.cuda.synchronize()
        assert torch.equal(h, he), f"replay {rep}: state differs"
        assert all(torch.equal(a, b) for a, b in zip(ys, ye)), f"replay {rep}: outputs differ"
        log(f"graph decode replay {rep}: bit-exact")


def test_graph_scan_and_ssd_replays_follow_new_inputs():
    s = inputs.make_scan_inputs(2, 300, 200, io="bf16", seed=(39, 7100), with_h0=True)
    t = {k: dev(getattr(s, k), "bf16") for k in ("x", "delta", "z", "B", "C")}
    p = {k: f32dev(getattr(s, k)) for k in ("A", "Dskip", "dt_bias", "h0")}
    ws = torch.empty(binding.workspace_bytes(2, 300, 200, 1, 64), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(t["x"])
    # an SSD shape cut into segments: the first pass, the fold and the layer are all captured
    assert binding.ssd_plan(1, 3000, 2, 128) == (2, 24)
    q = inputs.make_ssd_inputs(1, 3000, 2, seed=(39, 7101), with_h0=True)
    u = {k: dev(getattr(q, k), "bf16") for k in ("x", "delta", "z", "B", "C")}
    v = {k: f32dev(getattr(q, k)) for k in ("A", "Dskip", "dt_bias", "h0")}
    wss = torch.empty(binding.ssd_workspace_bytes(1, 3000, 2, 128), dtype=torch.uint8, device="cuda")
    ys = torch.empty_like(u["x"])

    res = {}

    def calls():
        _, res["h"] = binding.scan_fwd(t["x"], t["delta"], p["A"], t["B"], t["C"], p["Dskip"], p["dt_bias"],
                                       z=t["z"], h0=p["h0"], chunk_len=64, out=y, workspace=ws)
        binding.ssd_fwd(u["x"], u["delta"], v["A"], u["B"], u["C"], v["Dskip"], v["dt_bias"], z=u["z"],
                        h0=v["h0"], out=ys, workspace=wss, return_last_state=False)

    g = _capture(calls)
    hl = res["h"]                               # the captured call's h_L buffer (graph memory)
    rng = np.random.default_rng(7102)
    for rep in range(3):
        # new inputs written eagerly between replays
        t["x"].copy_(torch.from_numpy(rng.standard_normal(t["x"].shape, dtype=np.float32)).to("cuda"))
        u["x"].copy_(torch.from_numpy(rng.standard_normal(u["x"].shape, dtype=np.float32)).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yg, hg, ysg = y.clone(), hl.clone(), ys.clone()
        calls()                                # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(yg, y) and torch.equal(hg, res["h"]), f"replay {rep}: scan differs"
        assert torch.equal(ysg, ys), f"replay {rep}: ssd differs"
        log(f"graph scan + ssd replay {rep}: bit-exact")


def test_graph_backward_replays_match_eager():
    s = inputs.make_scan_inputs(2, 300, 200, io="bf16", seed=(39, 7200), with_h0=True)
    go = inputs.make_grad_outputs(2, 300, 200, io="bf16", seed=(39, 7200))
    t = {k: dev(getattr(s, k), "bf16") for k in ("x", "delta", "z", "B", "C")}
    p = {k: f32dev(getattr(s, k)) for k in ("A", "Dskip", "dt_bias", "h0")}
    dout, dh_last = dev(go.dout, "bf16"), f32dev(go.dh_last)
    ws = torch.empty(binding.bwd_workspace_bytes(2, 300, 200, 1, 64), dtype=torch.uint8, device="cuda")
    grads = binding.scan_bwd(t["x"], t["delta"], p["A"], t["B"], t["C"], p["Dskip"], p["dt_bias"], dout,
                             z=t["z"], h0=p["h0"], dh_last=dh_last, chunk_len=64, workspace=ws)

    def call(into):
        binding.scan_bwd(t["x"], t["delta"], p["A"], t["B"], t["C"], p["Dskip"], p["dt_bias"], dout, z=t["z"],
                         h0=p["h0"], dh_last=dh_last, chunk_len=64, workspace=ws, grads=into)

    g = _capture(lambda: call(grads))
    fresh = {k: (None if v is None else torch.empty_like(v)) for k, v in grads.items()}
    rng = np.random.default_rng(7201)
    for rep in range(3):
        dout.copy_(torch.from_numpy(rng.standard_normal(dout.shape, dtype=np.float32)).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(fresh)                            # eager, same inputs, separate outputs
        torch.cuda.synchronize()
        for k, v in grads.items():
            if v is not None:
                assert torch.equal(v, fresh[k]), f"replay {rep}: d{k} differs"
        log(f"graph backward replay {rep}: bit-exact over {sum(v is not None for v in grads.values())} gradients")
