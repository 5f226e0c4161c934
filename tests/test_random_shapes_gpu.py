"""Seeded random shapes for every entry point against the float64 oracle (needs an MI355X).

The hand-picked cases elsewhere pin the edges one at a time; these draw
(batch, L, D, chunk length, io dtype, gate, h0, ...) from a fixed seed so that
combinations nobody picked by hand are covered too: ragged chunks and tiles in
both directions, odd widths (16-bit loads), one-token sequences, every
convolution width, and all three SSD state sizes.  Each case prints its
parameters before it runs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL, assert_close, assert_grads_close, dev, gpu_bwd, gpu_conv_scan, gpu_scan, gpu_ssd,
                      host64, log, oracle_bwd, oracle_conv_scan, oracle_scan, oracle_ssd)
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu

CHUNKS = (0, 32, 64, 96, 160)


def _draw(kind, i):
    r = np.random.default_rng([39, 8000, kind, i])
    return dict(batch=int(r.integers(1, 5)), L=int(r.integers(1, 700)), D=int(r.integers(1, 300)),
                chunk=int(r.choice(CHUNKS)), io=str(r.choice(["bf16", "f32"])), gated=bool(r.integers(0, 2)),
                h0=bool(r.integers(0, 2)), K=int(r.integers(1, 5)), seed=8000 + 100 * kind + i)


@pytest.mark.parametrize("i", range(24))
def test_scan_random_shape(i):
    c = _draw(0, i)
    log(f"scan case {i}: {c}")
    s = inputs.make_scan_inputs(c["batch"], c["L"], c["D"], io=c["io"], seed=(39, c["seed"]), gated=c["gated"],
                                with_h0=c["h0"])
    y, h = gpu_scan(s, chunk_len=c["chunk"], h0=s.h0, gated=c["gated"])
    ry, rh = oracle_scan(s, h0=s.h0, gated=c["gated"])
    assert_close(host64(y), ry, TOL[c["io"]], f"scan case {i} y")
    assert_close(host64(h), rh, TOL[c["io"]], f"scan case {i} h_L")


@pytest.mark.parametrize("i", range(16))
def test_conv_scan_random_shape(i):
    c = _draw(1, i)
    log(f"conv scan case {i}: {c}")
    s = inputs.make_scan_inputs(c["batch"], c["L"], c["D"], io=c["io"], seed=(39, c["seed"]), gated=c["gated"],
                                with_h0=c["h0"])
    cp = inputs.make_conv_params(c["batch"], c["D"], c["K"], io=c["io"], seed=(39, c["seed"]),
                                 with_init=c["K"] > 1)
    y, h, _ = gpu_conv_scan(s, cp, chunk_len=c["chunk"], h0=s.h0, gated=c["gated"], conv_last=False)
    ry, rh = oracle_conv_scan(s, cp, h0=s.h0, gated=c["gated"])
    assert_close(host64(y), ry, TOL[c["io"]], f"conv scan case {i} y")
    assert_close(host64(h), rh, TOL[c["io"]], f"conv scan case {i} h_L")


@pytest.mark.parametrize("i", range(16))
def test_bwd_random_shape(i):
    c = _draw(2, i)
    c["L"] = min(c["L"], 400)
    log(f"bwd case {i}: {c}")
    s = inputs.make_scan_inputs(c["batch"], c["L"], c["D"], io=c["io"], seed=(39, c["seed"]), gated=c["gated"],
                                with_h0=c["h0"], A_random=True)
    go = inputs.make_grad_outputs(c["batch"], c["L"], c["D"], io=c["io"], seed=(39, c["seed"]), with_dh_last=True)
    g = gpu_bwd(s, go, chunk_len=c["chunk"], gated=c["gated"], h0=c["h0"])
    ref = oracle_bwd(s, go, gated=c["gated"], h0=c["h0"])
    assert_grads_close(g, ref, TOL[c["io"]], f"bwd case {i}")


@pytest.mark.parametrize("i", range(12))
def test_decode_random_shape(i):
    """A few chained decode steps (with and without the convolution) on a random (batch, D)."""
    c = _draw(3, i)
    batch, D, io, K = c["batch"] * 7, c["D"] * 3, c["io"], c["K"]
    conv = i % 2 == 1
    log(f"decode case {i}: batch {batch} D {D} io {io} conv K={K if conv else 0} gated {c['gated']}")
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D, seed=(39, c["seed"]))
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h, hs = f(h0), h0.astype(np.float64)
    cp = inputs.make_conv_params(batch, D, K, io=io, seed=(39, c["seed"]), with_init=K > 1) if conv else None
    cs = dev(cp.init, io) if (conv and K > 1) else None
    css = cp.init if (conv and K > 1) else (np.zeros((batch, 0, D), dtype=np.uint16 if io == "bf16" else np.float32)
                                           if conv else None)
    for step in range(3):
        tok = inputs.decode_token(step, batch, D, io=io, gated=c["gated"], seed_root=(39, c["seed"]))
        z = dev(tok.z, io) if c["gated"] else None
        if conv:
            y = binding.conv_state_update(h, cs, dev(tok.x, io), f(cp.w), f(cp.b), dev(tok.delta, io), f(A),
                                          dev(tok.B, io), dev(tok.C, io), f(Dskip), f(dt_bias), z=z)
            ry, hs, css = oracle.conv_state_update(css, hs, tok.x, cp.w, cp.b, tok.delta, A, tok.B, tok.C, Dskip,
                                                   dt_bias, z=tok.z if c["gated"] else None, io=io)
        else:
            y = binding.state_update(h, dev(tok.x, io), dev(tok.delta, io), f(A), dev(tok.B, io), dev(tok.C, io),
                                     f(Dskip), f(dt_bias), z=z)
            ry, hs = oracle.state_update(hs, tok.x, tok.delta, A, tok.B, tok.C, Dskip, dt_bias,
                                         z=tok.z if c["gated"] else None, io=io)
        torch.cuda.synchronize()
        assert_close(host64(y), ry, TOL[io], f"decode case {i} step {step} y")
        assert_close(host64(h), hs, TOL[io], f"decode case {i} step {step} h")


@pytest.mark.parametrize("i", range(12))
def test_ssd_random_shape(i):
    r = np.random.default_rng([39, 8000, 4, i])
    batch, L, H = int(r.integers(1, 3)), int(r.integers(1, 400)), int(r.integers(1, 6))
    N = int(r.choice([64, 128, 256]))
    gated, h0 = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    log(f"ssd case {i}: batch {batch} L {L} H {H} N {N} gated {gated} h0 {h0}")
    s = inputs.make_ssd_inputs(batch, L, H, N=N, seed=(39, 8400 + i), gated=gated, with_h0=h0)
    y, h = gpu_ssd(s, gated=gated, h0=h0)
    ry, rh = oracle_ssd(s, gated=gated, h0=h0)
    assert_close(host64(y), ry, TOL["bf16"], f"ssd case {i} y")
    assert_close(host64(h), rh, TOL["bf16"], f"ssd case {i} h_L")
