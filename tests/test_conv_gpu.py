"""The scan fed by the fused local convolution, on the GPU, against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, dev, gpu_conv_scan, host64, log, oracle_conv_scan
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,L,D,io,K,gated,h0,init,chunk", [
    (2, 300, 200, "bf16", 4, True, True, True, 64),     # 5 chunks, ragged tail, stream continued
    (1, 257, 130, "f32", 3, False, False, False, 32),   # 9 chunks, last holds one token
    (3, 97, 65, "bf16", 2, True, True, True, 32),       # odd D: 16-bit loads
    (1, 64, 64, "f32", 1, True, False, False, 64),      # width 1: a per-channel scale, bias and silu
    (1, 2, 16, "bf16", 4, True, False, True, 32),       # shorter than the window: conv_last keeps init rows
    (4, 512, 320, "bf16", 4, True, True, True, 0),      # automatic plan
])
def test_conv_scan_matches_oracle(batch, L, D, io, K, gated, h0, init, chunk):
    s = inputs.make_scan_inputs(batch, L, D, io=io, seed=(39, 5000 + L + D), gated=gated, with_h0=h0)
    cp = inputs.make_conv_params(batch, D, K, io=io, seed=(39, 5000 + L + D), with_init=init)
    log(f"conv scan {batch}x{L}x{D} {io} K={K} gated={gated} h0={h0} init={init} chunk {chunk}")
    y, h, cl = gpu_conv_scan(s, cp, chunk_len=chunk, h0=s.h0, gated=gated)
    ry, rh = oracle_conv_scan(s, cp, h0=s.h0, gated=gated)
    assert_close(host64(y), ry, TOL[io], f"conv scan {batch}x{L}x{D} y")
    assert_close(host64(h), rh, TOL[io], f"conv scan {batch}x{L}x{D} h_L")
    if K > 1:
        dec = (lambda a: oracle.decode(a, io))
        head = dec(cp.init) if cp.init is not None else np.zeros((batch, K - 1, D))
        ref_last = np.concatenate([head, dec(s.x)], axis=1)[:, -(K - 1):]
        assert np.array_equal(host64(cl), ref_last), "conv_last must be the last K-1 inputs, bit for bit"
    else:
        assert cl is None


def test_conv_scan_stream_split():
    """conv_scan over [0, L) = conv_scan over [0, L1) then [L1, L) from (h_L1, conv_last)."""
    io = "bf16"
    s = inputs.make_scan_inputs(2, 500, 192, io=io, seed=(39, 5100), with_h0=True)
    cp = inputs.make_conv_params(2, 192, 4, io=io, seed=(39, 5100), with_init=True)
    d = {k: dev(getattr(s, k), io) for k in ("x", "delta", "z", "B", "C")}
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, Dk, bias, w, b = f(s.A), f(s.Dskip), f(s.dt_bias), f(cp.w), f(cp.b)
    run = lambda sl, h0, init: binding.conv_scan_fwd(d["x"][:, sl].contiguous(), w, b, d["delta"][:, sl].contiguous(),
                                                     A, d["B"][:, sl].contiguous(), d["C"][:, sl].contiguous(), Dk,
                                                     bias, z=d["z"][:, sl].contiguous(), h0=h0, conv_init=init,
                                                     chunk_len=64, return_conv_last=True)
    y, h, cl = run(slice(None), f(s.h0), dev(cp.init, io))
    for L1 in (1, 64, 333):
        ya, ha, ca = run(slice(0, L1), f(s.h0), dev(cp.init, io))
        yb, hb, cb = run(slice(L1, None), ha, ca)
        torch.cuda.synchronize()
        assert_close(np.concatenate([host64(ya), host64(yb)], axis=1), host64(y), 1e-2, f"split {L1} y")
        assert_close(host64(hb), host64(h), 1e-5, f"split {L1} h_L")
        assert torch.equal(cb, cl)


def test_conv_scan_full_size_sampled():
    """The 130M-layer shape with a width-4 convolution, at the automatic plan, on 64 sampled channels."""
    s = inputs.make_workload("mamba-130m-layer")
    cp = inputs.make_conv_params(8, 1536, 4, io="bf16", seed=inputs.SCAN_WORKLOADS["mamba-130m-layer"]["seed"],
                                 with_init=False)
    y, h, _ = gpu_conv_scan(s, cp, conv_last=False)
    ch = np.random.default_rng([39, 5200]).choice(1536, size=64, replace=False)
    ry, rh = oracle_conv_scan(s, cp, channels=ch)
    assert_close(host64(y)[:, :, ch], ry, TOL["bf16"], "conv 130M layer y (sampled)")
    assert_close(host64(h)[:, ch], rh, TOL["bf16"], "conv 130M layer h_L (sampled)")


def test_conv_scan_errors():
    s = inputs.make_scan_inputs(1, 64, 64, io="bf16", seed=(39, 5300))
    x = dev(s.x, "bf16")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w5 = torch.zeros(64, 5, device="cuda")
    with pytest.raises(binding.SSMError) as e:
        binding.conv_scan_fwd(x, w5, f(np.zeros(64, np.float32)), x, f(s.A), dev(s.B, "bf16"), dev(s.C, "bf16"),
                              f(s.Dskip), f(s.dt_bias))
    assert e.value.status == -2


@pytest.mark.parametrize("batch,D,io,K,gated", [(3, 130, "bf16", 4, True), (9, 64, "f32", 2, False),
                                                 (17, 257, "bf16", 1, True), (1, 1, "bf16", 3, True)])
def test_conv_decode_step_matches_oracle(batch, D, io, K, gated):
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    tok = inputs.decode_token(4, batch, D, io=io, gated=gated)
    cp = inputs.make_conv_params(batch, D, K, io=io, seed=(39, 5400 + D), with_init=True)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h = f(h0)
    cs = dev(cp.init, io) if K > 1 else None
    y = binding.conv_state_update(h, cs, dev(tok.x, io), f(cp.w), f(cp.b), dev(tok.delta, io), f(A), dev(tok.B, io),
                                  dev(tok.C, io), f(Dskip), f(dt_bias), z=dev(tok.z, io) if gated else None)
    torch.cuda.synchronize()
    init = cp.init if K > 1 else np.zeros((batch, 0, D), dtype=tok.x.dtype)
    ry, rh, rcs = oracle.conv_state_update(init, h0, tok.x, cp.w, cp.b, tok.delta, A, tok.B, tok.C, Dskip, dt_bias,
                                           z=tok.z if gated else None, io=io)
    assert_close(host64(y), ry, TOL[io], f"conv decode {batch}x{D} K={K} y")
    assert_close(host64(h), rh, TOL[io], f"conv decode {batch}x{D} K={K} h")
    if K > 1:
        assert np.array_equal(host64(cs), oracle.decode(rcs, io)), "conv state must shift by one input exactly"


def test_conv_decode_256x5120_chain_sampled():
    """The decode-256x5120-conv workload (width 4): 8 chained steps on the full 256 x 5120
    state in the bench's launch configuration; y, the state and the conv state of a
    16 x 256 sample of (batch row, channel) pairs against the oracle's own float64 chain."""
    batch, D, io = 256, 5120, "bf16"
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    cp = inputs.make_conv_params(batch, D, 4, io=io, seed=inputs.DECODE_WORKLOAD["seed"], with_init=True)
    r = np.random.default_rng([39, 5600])
    bsel = np.sort(np.concatenate([[0, batch - 1], r.choice(np.arange(1, batch - 1), 14, replace=False)]))
    dsel = np.sort(np.concatenate([[0, 63, 64, D - 1], r.choice(np.arange(65, D - 1), 252, replace=False)]))
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h, cs = f(h0), dev(cp.init, io)
    tA, tD, tb, w, b = f(A), f(Dskip), f(dt_bias), f(cp.w), f(cp.b)
    sub = lambda a: a[bsel][:, dsel]
    hs = sub(h0).astype(np.float64)
    css = cp.init[bsel][:, :, dsel]
    for step in range(8):
        tok = inputs.decode_token(step, batch, D)
        y = binding.conv_state_update(h, cs, dev(tok.x, io), w, b, dev(tok.delta, io), tA, dev(tok.B, io),
                                      dev(tok.C, io), tD, tb, z=dev(tok.z, io))
        torch.cuda.synchronize()
        ry, hs, css = oracle.conv_state_update(css, hs, sub(tok.x), cp.w[dsel], cp.b[dsel], sub(tok.delta), A[dsel],
                                               tok.B[bsel], tok.C[bsel], Dskip[dsel], dt_bias[dsel], z=sub(tok.z),
                                               io=io)
        assert_close(sub(host64(y)), ry, TOL[io], f"conv decode step {step} y")
        assert_close(sub(host64(h)), hs, TOL[io], f"conv decode step {step} h")
        assert np.array_equal(host64(cs)[bsel][:, :, dsel], oracle.decode(css, io)), f"conv state at step {step}"


def test_conv_prompt_then_decode_equals_scan():
    """Serving a stream: conv scan over a prompt, then chained conv decode steps from its
    (h_last, conv_last), equal the conv scan over the whole sequence (oracle)."""
    io, batch, L, P, D = "bf16", 2, 120, 100, 96
    s = inputs.make_scan_inputs(batch, L, D, io=io, seed=(39, 5500), with_h0=True)
    cp = inputs.make_conv_params(batch, D, 4, io=io, seed=(39, 5500), with_init=True)
    d = {k: dev(getattr(s, k), io) for k in ("x", "delta", "z", "B", "C")}
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    A, Dk, bias, w, b = f(s.A), f(s.Dskip), f(s.dt_bias), f(cp.w), f(cp.b)
    sl = lambda k: d[k][:, :P].contiguous()
    _, h, cs = binding.conv_scan_fwd(sl("x"), w, b, sl("delta"), A, sl("B"), sl("C"), Dk, bias, z=sl("z"),
                                     h0=f(s.h0), conv_init=dev(cp.init, io), chunk_len=32, return_conv_last=True)
    outs = []
    for t in range(P, L):
        tk = lambda k: d[k][:, t].contiguous()
        outs.append(binding.conv_state_update(h, cs, tk("x"), w, b, tk("delta"), A, tk("B"), tk("C"), Dk, bias,
                                              z=tk("z")))
    yd = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    ry, rh = oracle_conv_scan(s, cp, h0=s.h0)
    assert_close(host64(yd), ry[:, P:], TOL[io], "prompt + decode y")
    assert_close(host64(h), rh, TOL[io], "prompt + decode h")
