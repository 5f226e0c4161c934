"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its binding, run the oracle on the same bits, compare."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from selective_state_space_39_amd import binding, inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}     # max|err| <= TOL * max|ref|


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, io, device="cuda"):
    """numpy io storage -> torch tensor on the GPU (bf16 bit patterns keep their bits)."""
    if a is None:
        return None
    if io == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def f32dev(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def gpu_scan(s: inputs.ScanInputs, chunk_len=0, h0=None, gated=True, want_h=True):
    io = s.io
    y, h = binding.scan_fwd(dev(s.x, io), dev(s.delta, io), f32dev(s.A), dev(s.B, io), dev(s.C, io),
                            f32dev(s.Dskip), f32dev(s.dt_bias), z=dev(s.z, io) if gated else None,
                            h0=f32dev(h0), chunk_len=chunk_len, return_last_state=want_h)
    torch.cuda.synchronize()
    return y, h


def oracle_scan(s: inputs.ScanInputs, channels=None, h0=None, gated=True):
    sel = slice(None) if channels is None else np.asarray(channels)
    x, dl = s.x[:, :, sel], s.delta[:, :, sel]
    z = s.z[:, :, sel] if (gated and s.z is not None) else None
    hh = None if h0 is None else h0[:, sel]
    return oracle.scan_fwd(x, dl, s.A[sel], s.B, s.C, s.Dskip[sel], s.dt_bias[sel], z=z, h0=hh, io=s.io)


def rel_err(a, ref):
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref))) / max(scale, 1e-300), scale


def assert_close(a, ref, tol, what):
    e, scale = rel_err(a, ref)
    log(f"{what}: max|err|/max|ref| = {e:.3e} (max|ref| {scale:.3e}, bound {tol:.0e})")
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: {e:.3e} > {tol:.0e}"
    return e


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

GRAD_KEYS = ("x", "delta", "z", "B", "C", "A", "Dskip", "dt_bias", "h0")


def gpu_bwd(s: inputs.ScanInputs, go: inputs.GradOutputs, chunk_len=0, gated=True, h0=True, want_dh0=True):
    io = s.io
    g = binding.scan_bwd(dev(s.x, io), dev(s.delta, io), f32dev(s.A), dev(s.B, io), dev(s.C, io),
                         f32dev(s.Dskip), f32dev(s.dt_bias), dev(go.dout, io),
                         z=dev(s.z, io) if gated else None, h0=f32dev(s.h0) if h0 else None,
                         dh_last=f32dev(go.dh_last), chunk_len=chunk_len, want_dh0=want_dh0)
    torch.cuda.synchronize()
    return g


def oracle_bwd(s: inputs.ScanInputs, go: inputs.GradOutputs, gated=True, h0=True, strip=None):
    """oracle.scan_bwd on the same bits; with `strip`, channel strips at a time (dB and dC summed)."""
    D = s.x.shape[2]
    strip = strip or D
    out = None
    for d0 in range(0, D, strip):
        sel = slice(d0, min(D, d0 + strip))
        r = oracle.scan_bwd(s.x[:, :, sel], s.delta[:, :, sel], s.A[sel], s.B, s.C, s.Dskip[sel], s.dt_bias[sel],
                            go.dout[:, :, sel], z=s.z[:, :, sel] if gated else None,
                            h0=s.h0[:, sel] if (h0 and s.h0 is not None) else None,
                            dh_last=None if go.dh_last is None else go.dh_last[:, sel], io=s.io)
        if out is None:
            out = {k: (None if v is None else [v]) for k, v in r.items()}
            continue
        for k, v in r.items():
            if v is not None:
                out[k].append(v)
    axis = {"x": 2, "delta": 2, "z": 2, "A": 0, "Dskip": 0, "dt_bias": 0, "h0": 1}
    res = {}
    for k, parts in out.items():
        if parts is None:
            res[k] = None
        elif k in ("B", "C"):
            res[k] = np.sum(parts, axis=0)
        else:
            res[k] = np.concatenate(parts, axis=axis[k])
    return res


def assert_grads_close(g, ref, tol, what, keys=GRAD_KEYS):
    for k in keys:
        if ref.get(k) is None:
            assert g.get(k) is None, f"{what}: d{k} should be absent"
            continue
        assert_close(host64(g[k]), ref[k], tol, f"{what} d{k}")


# ---------------------------------------------------------------------------
# the scan fed by the local convolution
# ---------------------------------------------------------------------------

def gpu_conv_scan(s: inputs.ScanInputs, cp: inputs.ConvParams, chunk_len=0, h0=None, gated=True, conv_last=True):
    io = s.io
    y, h, cl = binding.conv_scan_fwd(dev(s.x, io), f32dev(cp.w), f32dev(cp.b), dev(s.delta, io), f32dev(s.A),
                                     dev(s.B, io), dev(s.C, io), f32dev(s.Dskip), f32dev(s.dt_bias),
                                     z=dev(s.z, io) if gated else None, h0=f32dev(h0),
                                     conv_init=dev(cp.init, io), chunk_len=chunk_len, return_conv_last=conv_last)
    torch.cuda.synchronize()
    return y, h, cl


def oracle_conv_scan(s: inputs.ScanInputs, cp: inputs.ConvParams, channels=None, h0=None, gated=True):
    sel = slice(None) if channels is None else np.asarray(channels)
    z = s.z[:, :, sel] if (gated and s.z is not None) else None
    init = None if cp.init is None else cp.init[:, :, sel]
    hh = None if h0 is None else h0[:, sel]
    return oracle.conv_scan_fwd(s.x[:, :, sel], cp.w[sel], cp.b[sel], s.delta[:, :, sel], s.A[sel], s.B, s.C,
                                s.Dskip[sel], s.dt_bias[sel], z=z, h0=hh, conv_init=init, io=s.io)


# ---------------------------------------------------------------------------
# SSD layer
# ---------------------------------------------------------------------------

def gpu_ssd(s, gated=True, h0=True):
    io = s.io
    y, h = binding.ssd_fwd(dev(s.x, io), dev(s.delta, io), f32dev(s.A), dev(s.B, io), dev(s.C, io),
                           f32dev(s.Dskip), f32dev(s.dt_bias), z=dev(s.z, io) if gated else None,
                           h0=f32dev(s.h0) if h0 else None)
    torch.cuda.synchronize()
    return y, h


def oracle_ssd(s, heads=None, gated=True, h0=True):
    sel = slice(None) if heads is None else np.asarray(heads)
    z = s.z[:, :, sel] if (gated and s.z is not None) else None
    hh = s.h0[:, sel] if (h0 and s.h0 is not None) else None
    return oracle.ssd_fwd(s.x[:, :, sel], s.delta[:, :, sel], s.A[sel], s.B, s.C, s.Dskip[sel], s.dt_bias[sel],
                          z=z, h0=hh, io=s.io)
