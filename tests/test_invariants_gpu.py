"""GPU invariants of the scan and decode kernels (needs an MI355X).

Every case is compared with the float64 oracle at the io tolerance, and some
identities are checked between GPU results themselves.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, dev, f32dev, gpu_scan, host64, log, oracle_scan
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _dev_all(s):
    io = s.io
    return dict(x=dev(s.x, io), delta=dev(s.delta, io), z=dev(s.z, io), B=dev(s.B, io), C=dev(s.C, io),
                A=f32dev(s.A), D=f32dev(s.Dskip), dt_bias=f32dev(s.dt_bias), h0=f32dev(s.h0))


def _run(t, chunk_len=0, gated=True, h0=True, **kw):
    y, h = binding.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"],
                            z=t["z"] if gated else None, h0=t["h0"] if h0 else None, chunk_len=chunk_len, **kw)
    torch.cuda.synchronize()
    return y, h


@pytest.mark.parametrize("chunk_len", [32, 64, 96, 160, 512, 1024])
def test_chunk_length_invariance(chunk_len):
    """Any chunk length gives the oracle's answer (ragged last chunk included)."""
    s = inputs.make_scan_inputs(2, 777, 192, io="bf16", seed=(39, 2001), with_h0=True)
    t = _dev_all(s)
    log(f"chunk_len {chunk_len}: plan {binding.plan(2, 777, 192, 1, chunk_len)}")
    y, h = _run(t, chunk_len)
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(y), ry, TOL["bf16"], f"chunk {chunk_len} y")
    assert_close(host64(h), rh, TOL["bf16"], f"chunk {chunk_len} h_L")


def test_bitwise_determinism():
    s = inputs.make_scan_inputs(4, 512, 320, io="bf16", seed=(39, 2002), with_h0=True)
    t = _dev_all(s)
    y1, h1 = _run(t, 64)
    y2, h2 = _run(t, 64)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_split_resume_on_gpu():
    """scan(0:L) == scan(L1:L, h0 = h_L1) after scan(0:L1), all on the GPU."""
    s = inputs.make_scan_inputs(2, 600, 130, io="f32", seed=(39, 2003), with_h0=True)
    t = _dev_all(s)
    y, h = _run(t, 64)
    L1 = 257
    part = lambda k, sl: t[k][:, sl].contiguous()
    t1 = dict(t, x=part("x", slice(0, L1)), delta=part("delta", slice(0, L1)), z=part("z", slice(0, L1)),
              B=part("B", slice(0, L1)), C=part("C", slice(0, L1)))
    ya, ha = _run(t1, 64)
    t2 = dict(t, x=part("x", slice(L1, None)), delta=part("delta", slice(L1, None)), z=part("z", slice(L1, None)),
              B=part("B", slice(L1, None)), C=part("C", slice(L1, None)), h0=ha)
    yb, hb = _run(t2, 96)
    ref = host64(y)
    assert_close(np.concatenate([host64(ya), host64(yb)], axis=1), ref, TOL["f32"], "split y vs whole")
    assert_close(host64(hb), host64(h), TOL["f32"], "split h_L vs whole")


def test_scan_equals_chained_decode_on_gpu():
    s = inputs.make_scan_inputs(3, 24, 96, io="bf16", seed=(39, 2004), with_h0=True)
    t = _dev_all(s)
    y, h = _run(t, 0)
    hs = t["h0"].clone()
    outs = []
    for k in range(s.x.shape[1]):
        outs.append(binding.state_update(hs, t["x"][:, k].contiguous(), t["delta"][:, k].contiguous(), t["A"],
                                         t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"],
                                         t["dt_bias"], z=t["z"][:, k].contiguous()))
    yd = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(yd), ry, TOL["bf16"], "chained decode y")
    assert_close(host64(hs), rh, TOL["bf16"], "chained decode h")
    # the two GPU routes agree with each other to fp32 state accuracy
    assert_close(host64(hs), host64(h), 1e-5, "decode chain vs scan state")


@pytest.mark.parametrize("bias,what", [(-60.0, "pass-through"), (200.0, "overwrite")])
def test_forget_gate_limits(bias, what):
    """dt_bias = -60: the state is untouched and out = D x silu(z); +200: the state is overwritten."""
    s = inputs.make_scan_inputs(2, 300, 128, io="bf16", seed=(39, 2005), with_h0=True)
    s.dt_bias = np.full_like(s.dt_bias, bias)
    t = _dev_all(s)
    y, h = _run(t, 64)
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(y), ry, TOL["bf16"], f"{what} y")
    assert_close(host64(h), rh, TOL["bf16"], f"{what} h_L")
    if bias < 0:
        # the carried state decays by exp(A * ~1e-26) = 1 in fp32: h_L is h0 exactly
        assert torch.equal(h, t["h0"])


def test_outputs_fully_written_over_nan_poison():
    """y, h_L and the workspace start as NaN: every output is written, no stale workspace value leaks."""
    s = inputs.make_scan_inputs(2, 500, 200, io="bf16", seed=(39, 2006), with_h0=True)
    t = _dev_all(s)
    y = torch.full_like(t["x"], float("nan"))
    nws = binding.workspace_bytes(2, 500, 200, binding.SSM_BF16, 64)
    ws = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    y2, h2 = _run(t, 64, out=y, workspace=ws)
    assert y2.data_ptr() == y.data_ptr()
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(y), ry, TOL["bf16"], "poisoned y")
    assert_close(host64(h2), rh, TOL["bf16"], "poisoned h_L")


@pytest.mark.parametrize("batch,L,D,io,gated,h0", [
    (1, 1, 1, "bf16", True, False),
    (1, 5, 1, "f32", False, True),
    (3, 97, 65, "bf16", True, True),      # odd D: 16-bit load path
    (2, 64, 63, "bf16", False, True),
    (1, 33, 2, "bf16", True, True),
    (5, 131, 257, "f32", True, False),
])
def test_odd_shapes(batch, L, D, io, gated, h0):
    s = inputs.make_scan_inputs(batch, L, D, io=io, seed=(39, 3000 + L + D), gated=gated, with_h0=h0)
    y, h = gpu_scan(s, chunk_len=32, h0=s.h0, gated=gated)
    ry, rh = oracle_scan(s, h0=s.h0, gated=gated)
    assert_close(host64(y), ry, TOL[io], f"odd {batch}x{L}x{D} y")
    assert_close(host64(h), rh, TOL[io], f"odd {batch}x{L}x{D} h_L")


def test_misaligned_inputs_use_16bit_loads():
    """bf16 io that is 2- but not 4-byte aligned (a view one element in) still matches."""
    s = inputs.make_scan_inputs(2, 200, 128, io="bf16", seed=(39, 2007))
    io = "bf16"

    def shifted(a):
        flat = dev(np.concatenate([np.zeros(1, np.uint16), a.reshape(-1)]), io)
        return flat[1:].view(a.shape)

    x, dl, z = shifted(s.x), shifted(s.delta), shifted(s.z)
    assert x.data_ptr() % 4 == 2
    y, h = binding.scan_fwd(x, dl, f32dev(s.A), dev(s.B, io), dev(s.C, io), f32dev(s.Dskip), f32dev(s.dt_bias),
                            z=z, chunk_len=64)
    torch.cuda.synchronize()
    ry, rh = oracle_scan(s)
    assert_close(host64(y), ry, TOL["bf16"], "misaligned y")
    assert_close(host64(h), rh, TOL["bf16"], "misaligned h_L")


def test_no_last_state_requested():
    s = inputs.make_scan_inputs(2, 300, 256, io="bf16", seed=(39, 2008))
    t = _dev_all(s)
    y, h = _run(t, 64, h0=False, return_last_state=False)
    assert h is None
    ry, _ = oracle_scan(s)
    assert_close(host64(y), ry, TOL["bf16"], "no h_L y")


@pytest.mark.parametrize("batch,D,io,gated", [(3, 130, "bf16", True), (9, 64, "f32", False), (1, 1, "bf16", True),
                                              (17, 257, "bf16", False)])
def test_decode_shapes(batch, D, io, gated):
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    tok = inputs.decode_token(3, batch, D, io=io, gated=gated)
    h = f32dev(h0)
    y = binding.state_update(h, dev(tok.x, io), dev(tok.delta, io), f32dev(A), dev(tok.B, io), dev(tok.C, io),
                             f32dev(Dskip), f32dev(dt_bias), z=dev(tok.z, io) if gated else None)
    torch.cuda.synchronize()
    ry, rh = oracle.state_update(h0, tok.x, tok.delta, A, tok.B, tok.C, Dskip, dt_bias,
                                 z=tok.z if gated else None, io=io)
    assert_close(host64(y), ry, TOL[io], f"decode {batch}x{D} y")
    assert_close(host64(h), rh, TOL[io], f"decode {batch}x{D} h")


@pytest.mark.parametrize("io,gated", [("bf16", True), ("f32", False)])
def test_decode_unaligned_bc_uses_element_loads(io, gated):
    """B and C one element into their buffers (aligned for their element, not for a 4-element
    vector) take the element-by-element path of the decode step and give the same result as the
    oracle; the aligned copies (vector path) agree with it bit for bit."""
    batch, D = 11, 200
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, D)
    tok = inputs.decode_token(5, batch, D, io=io, gated=gated)

    def shifted(a):
        pad = np.zeros(1, np.uint16 if io == "bf16" else np.float32)
        flat = dev(np.concatenate([pad, np.ascontiguousarray(a).reshape(-1)]), io)
        return flat[1:].view(a.shape)

    B1, C1 = shifted(tok.B), shifted(tok.C)
    esz = 2 if io == "bf16" else 4
    assert B1.data_ptr() % (4 * esz) != 0 and C1.data_ptr() % (4 * esz) != 0
    args = (dev(tok.x, io), dev(tok.delta, io), f32dev(A))
    rest = (f32dev(Dskip), f32dev(dt_bias))
    z = dev(tok.z, io) if gated else None
    h_u, h_a = f32dev(h0), f32dev(h0)
    y_u = binding.state_update(h_u, *args, B1, C1, *rest, z=z)
    y_a = binding.state_update(h_a, *args, dev(tok.B, io), dev(tok.C, io), *rest, z=z)
    torch.cuda.synchronize()
    ry, rh = oracle.state_update(h0, tok.x, tok.delta, A, tok.B, tok.C, Dskip, dt_bias,
                                 z=tok.z if gated else None, io=io)
    assert_close(host64(y_u), ry, TOL[io], "unaligned B, C decode y")
    assert_close(host64(h_u), rh, TOL[io], "unaligned B, C decode h")
    assert torch.equal(y_u, y_a) and torch.equal(h_u, h_a)


def test_errors_raise_before_launch():
    s = inputs.make_scan_inputs(1, 64, 64, io="bf16", seed=(39, 2009))
    t = _dev_all(s)
    with pytest.raises(binding.SSMError) as e:
        binding.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], out=t["x"])
    assert e.value.status == -7
    with pytest.raises(binding.SSMError):
        binding.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], chunk_len=48)


def test_nonfinite_inputs_propagate():
    """A NaN in x reaches y at that token onward (through the state) and h_L; other rows stay finite."""
    s = inputs.make_scan_inputs(2, 200, 64, io="f32", seed=(39, 2010))
    s.x = s.x.copy()
    s.x[0, 50, 3] = np.nan
    y, h = gpu_scan(s, chunk_len=64)
    yh, hh = host64(y), host64(h)
    assert np.all(np.isfinite(yh[1])) and np.all(np.isfinite(hh[1])), "batch row 1 must stay finite"
    assert np.all(np.isfinite(yh[0, :50])), "tokens before the NaN are unaffected"
    assert np.isnan(yh[0, 50:, 3]).all(), "the NaN propagates through channel 3's state"
    assert np.all(np.isfinite(np.delete(yh[0], 3, axis=1))), "other channels of row 0 stay finite"
    assert np.isnan(hh[0, 3]).all()


def test_side_stream():
    """Calls enqueue on torch's current stream: a scan on a side stream matches the default-stream result."""
    s = inputs.make_scan_inputs(2, 300, 130, io="bf16", seed=(39, 2011), with_h0=True)
    t = _dev_all(s)
    y0, h0 = _run(t, 64)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1, h1 = binding.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], z=t["z"],
                                  h0=t["h0"], chunk_len=64)
    side.synchronize()
    assert torch.equal(y0, y1) and torch.equal(h0, h1)


def test_concurrent_host_threads_on_own_streams():
    """Four host threads, each on a stream of its own, interleave scans, decode steps and SSD layers on their own
    inputs; every result equals, bit for bit, the same call made alone.  The library keeps no per-call state
    outside its arguments (the error string is per thread), so calls on different streams do not interact."""
    import threading

    cases = []
    for k in range(4):
        s = inputs.make_scan_inputs(2, 333 + 40 * k, 96 + 32 * k, io="bf16", seed=(39, 2100 + k), with_h0=True)
        q = inputs.make_ssd_inputs(1, 150 + 30 * k, 3, N=(64, 128, 256, 128)[k], seed=(39, 2110 + k), with_h0=True)
        A, Dskip, dt_bias, h0 = inputs.decode_params(8, 256, seed=(39, 2120 + k))
        tok = inputs.decode_token(0, 8, 256, io="bf16", seed_root=(39, 2120 + k))
        cases.append((_dev_all(s), q, (f32dev(A), f32dev(Dskip), f32dev(dt_bias), h0, tok)))

    def one_round(case):
        t, q, (A, Dskip, dt_bias, h0, tok) = case
        y, h = binding.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], z=t["z"],
                                h0=t["h0"])
        qd = {k: dev(getattr(q, k), "bf16") for k in ("x", "delta", "z", "B", "C")}
        qy, qh = binding.ssd_fwd(qd["x"], qd["delta"], f32dev(q.A), qd["B"], qd["C"], f32dev(q.Dskip),
                                 f32dev(q.dt_bias), z=qd["z"], h0=f32dev(q.h0))
        hs = f32dev(h0)
        dy = binding.state_update(hs, dev(tok.x, "bf16"), dev(tok.delta, "bf16"), A, dev(tok.B, "bf16"),
                                  dev(tok.C, "bf16"), Dskip, dt_bias, z=dev(tok.z, "bf16"))
        return [y, h, qy, qh, dy, hs]

    alone = []
    for case in cases:
        alone.append(one_round(case))
        torch.cuda.synchronize()

    got, errors = [None] * len(cases), []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(5):
                    out = one_round(cases[i])
                st.synchronize()
            got[i] = out
        except Exception as e:      # reported below, on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    names = ["scan y", "scan h_L", "ssd y", "ssd h_L", "decode y", "decode h"]
    for i in range(len(cases)):
        for n, a, b in zip(names, alone[i], got[i]):
            assert torch.equal(a, b), f"thread {i}: {n} differs from the call made alone"
    log("4 threads x 5 rounds of scan, SSD and decode calls: all equal to the calls made alone")
