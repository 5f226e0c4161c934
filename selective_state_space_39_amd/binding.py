"""ctypes binding of libssm_scan.so over torch tensors.

Argument marshalling only: shapes and dtypes are checked, outputs and the
workspace are allocated with torch on the input's device, and every step of
the computation runs in the library's HIP kernels on torch's current stream.
Raises if the library is missing; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssm_scan.so")
ABI_VERSION = 2
N_STATE = 16
SSM_F32, SSM_BF16 = 0, 1

_lib = None


class SSMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"ssm_scan error {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m selective_state_space_39_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.ssm_abi_version.restype = i32
    L.ssm_abi_version.argtypes = []
    L.ssm_last_error.restype = ctypes.c_char_p
    L.ssm_last_error.argtypes = []
    L.ssm_scan_fwd_workspace_bytes.restype = i64
    L.ssm_scan_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i64]
    L.ssm_scan_fwd_plan.restype = i32
    L.ssm_scan_fwd_plan.argtypes = [i64, i64, i64, i64, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ssm_scan_fwd.restype = i32
    L.ssm_scan_fwd.argtypes = [vp] * 11 + [i64, i64, i64, i64, i32, i64, vp, i64, vp]
    L.ssm_scan_fwd_noalloc.restype = i32
    L.ssm_scan_fwd_noalloc.argtypes = [vp] * 11 + [i64, i64, i64, i64, i32, i64, vp]
    L.ssm_conv_scan_fwd.restype = i32
    L.ssm_conv_scan_fwd.argtypes = [vp, vp, vp, i64, vp] + [vp] * 11 + [i64, i64, i64, i64, i32, i64, vp, i64, vp]
    L.ssm_conv_state_update.restype = i32
    L.ssm_conv_state_update.argtypes = [vp] * 5 + [i64] + [vp] * 8 + [i64, i64, i64, i32, vp]
    L.ssm_ssd_fwd.restype = i32
    L.ssm_ssd_fwd.argtypes = [vp] * 11 + [i64, i64, i64, i64, i64, i32, vp, i64, vp]
    L.ssm_ssd_fwd_workspace_bytes.restype = i64
    L.ssm_ssd_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.ssm_ssd_fwd_plan.restype = i32
    L.ssm_ssd_fwd_plan.argtypes = [i64, i64, i64, i64, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ssm_scan_bwd_workspace_bytes.restype = i64
    L.ssm_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i64]
    L.ssm_scan_bwd_plan.restype = i32
    L.ssm_scan_bwd_plan.argtypes = [i64, i64, i64, i64, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.ssm_scan_bwd.restype = i32
    L.ssm_scan_bwd.argtypes = [vp] * 20 + [i64, i64, i64, i64, i32, i64, vp, i64, vp]
    L.ssm_state_update.restype = i32
    L.ssm_state_update.argtypes = [vp] * 10 + [i64, i64, i64, i32, vp]
    L.ssm_timing_enable.restype = i32
    L.ssm_timing_enable.argtypes = [i32, ctypes.c_char_p]
    L.ssm_timing_collect.restype = i32
    L.ssm_timing_collect.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i64),
                                     ctypes.POINTER(ctypes.c_double)]
    if L.ssm_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {L.ssm_abi_version()}, expected {ABI_VERSION}")
    _lib = L
    return L


def abi_version() -> int:
    return lib().ssm_abi_version()


def _check(rc: int):
    if rc != 0:
        raise SSMError(rc, lib().ssm_last_error().decode())


def _io(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    if t.dtype == torch.float32:
        return SSM_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(batch: int, L: int, D: int, io_dtype: int = SSM_BF16, chunk_len: int = 0) -> int:
    n = lib().ssm_scan_fwd_workspace_bytes(batch, L, D, N_STATE, io_dtype, chunk_len)
    if n < 0:
        _check(int(n))
    return int(n)


def plan(batch: int, L: int, D: int, io_dtype: int = SSM_BF16, chunk_len: int = 0) -> Tuple[int, int]:
    """(chunk length, number of chunks) the library uses for this shape."""
    cl, nc = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ssm_scan_fwd_plan(batch, L, D, N_STATE, io_dtype, chunk_len, ctypes.byref(cl), ctypes.byref(nc)))
    return cl.value, nc.value


def scan_fwd(x, delta, A, B, C, D, dt_bias, z=None, h0=None, chunk_len: int = 0,
             return_last_state: bool = True, out=None, workspace=None):
    """Selective scan over whole sequences.

    x, delta, z: (batch, L, D); B, C: (batch, L, 16), all bfloat16 or all
    float32; A: (D, 16), D and dt_bias: (D,), h0: (batch, D, 16) float32.
    Returns (y, h_last) (h_last is None when return_last_state is False).
    """
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, D)")
    batch, L, Dc = x.shape
    dev = x.device
    io = _io(x)
    dt = x.dtype
    _need(x, "x", (batch, L, Dc), dt, dev)
    _need(delta, "delta", (batch, L, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, L, Dc), dt, dev)
    _need(B, "B", (batch, L, N_STATE), dt, dev)
    _need(C, "C", (batch, L, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, Dc, N_STATE), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", (batch, L, Dc), dt, dev)
    h_last = torch.empty((batch, Dc, N_STATE), dtype=torch.float32, device=dev) if return_last_state else None
    nws = workspace_bytes(batch, L, Dc, io, chunk_len)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nws:
        raise ValueError(f"workspace too small: {nws} bytes needed")
    rc = lib().ssm_scan_fwd(_ptr(x), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias),
                            _ptr(h0), _ptr(y), _ptr(h_last), batch, L, Dc, N_STATE, io, chunk_len,
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return y, h_last


def scan_fwd_noalloc(x, delta, A, B, C, D, dt_bias, z=None, h0=None, chunk_len: int = 0, out=None,
                     h_last_out=None, return_last_state: bool = True):
    """scan_fwd through ssm_scan_fwd_noalloc: no workspace, the chunk carries
    go to the library's fixed per-GPU scratch.  Pass `out` (and `h_last_out`)
    to allocate nothing here either.  Returns (y, h_last)."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, D)")
    batch, L, Dc = x.shape
    dev = x.device
    io = _io(x)
    dt = x.dtype
    _need(x, "x", (batch, L, Dc), dt, dev)
    _need(delta, "delta", (batch, L, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, L, Dc), dt, dev)
    _need(B, "B", (batch, L, N_STATE), dt, dev)
    _need(C, "C", (batch, L, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, Dc, N_STATE), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", (batch, L, Dc), dt, dev)
    h_last = None
    if return_last_state:
        h_last = (torch.empty((batch, Dc, N_STATE), dtype=torch.float32, device=dev) if h_last_out is None
                  else h_last_out)
        _need(h_last, "h_last_out", (batch, Dc, N_STATE), torch.float32, dev)
    rc = lib().ssm_scan_fwd_noalloc(_ptr(x), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
                                    _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last), batch, L, Dc, N_STATE, io,
                                    chunk_len, _stream(dev))
    _check(rc)
    return y, h_last


def conv_scan_fwd(xin, conv_w, conv_b, delta, A, B, C, D, dt_bias, z=None, h0=None, conv_init=None,
                  chunk_len: int = 0, return_last_state: bool = True, return_conv_last: bool = False,
                  out=None, workspace=None):
    """The scan fed by the fused local convolution: x = silu(causal depthwise conv(xin) + conv_b).

    conv_w: (D, K) float32 with K = 1..4; conv_b: (D,) float32; conv_init:
    (batch, K-1, D) like xin or None.  Returns (y, h_last, conv_last) with
    conv_last (batch, K-1, D) only when return_conv_last (else None).
    """
    if xin.dim() != 3:
        raise ValueError("xin must be (batch, L, D)")
    batch, L, Dc = xin.shape
    dev = xin.device
    io = _io(xin)
    dt = xin.dtype
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be (D, K)")
    K = conv_w.shape[1]
    _need(conv_w, "conv_w", (Dc, K), torch.float32, dev)
    _need(conv_b, "conv_b", (Dc,), torch.float32, dev)
    for t, name in ((xin, "xin"), (delta, "delta")):
        _need(t, name, (batch, L, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, L, Dc), dt, dev)
    _need(B, "B", (batch, L, N_STATE), dt, dev)
    _need(C, "C", (batch, L, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, Dc, N_STATE), torch.float32, dev)
    if conv_init is not None:
        _need(conv_init, "conv_init", (batch, K - 1, Dc), dt, dev)
    y = torch.empty_like(xin) if out is None else out
    _need(y, "out", (batch, L, Dc), dt, dev)
    h_last = torch.empty((batch, Dc, N_STATE), dtype=torch.float32, device=dev) if return_last_state else None
    conv_last = torch.empty((batch, K - 1, Dc), dtype=dt, device=dev) if (return_conv_last and K > 1) else None
    nws = workspace_bytes(batch, L, Dc, io, chunk_len)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nws:
        raise ValueError(f"workspace too small: {nws} bytes needed")
    rc = lib().ssm_conv_scan_fwd(_ptr(xin), _ptr(conv_w), _ptr(conv_b), K, _ptr(conv_init), _ptr(delta), _ptr(z),
                                 _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last),
                                 _ptr(conv_last), batch, L, Dc, N_STATE, io, chunk_len, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return y, h_last, conv_last


def bwd_workspace_bytes(batch: int, L: int, D: int, io_dtype: int = SSM_BF16, chunk_len: int = 0) -> int:
    n = lib().ssm_scan_bwd_workspace_bytes(batch, L, D, N_STATE, io_dtype, chunk_len)
    if n < 0:
        _check(int(n))
    return int(n)


def bwd_plan(batch: int, L: int, D: int, io_dtype: int = SSM_BF16, chunk_len: int = 0) -> Tuple[int, int]:
    """(chunk length, number of chunks) of the backward for this shape."""
    cl, nc = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ssm_scan_bwd_plan(batch, L, D, N_STATE, io_dtype, chunk_len, ctypes.byref(cl), ctypes.byref(nc)))
    return cl.value, nc.value


BWD_OUTPUTS = ("x", "delta", "z", "B", "C", "A", "Dskip", "dt_bias", "h0")


def scan_bwd(x, delta, A, B, C, D, dt_bias, dout, z=None, h0=None, dh_last=None, chunk_len: int = 0,
             want_dh0: bool = True, workspace=None, grads=None):
    """Gradients of sum(dout * out) + sum(dh_last * h_last) for scan_fwd with the same inputs.

    Returns a dict keyed by input name: "x", "delta", "z" (io dtype, "z" None
    when ungated), "B", "C" (batch, L, 16), "A" (D, 16), "Dskip", "dt_bias"
    (D,), all float32, and "h0" (batch, D, 16) float32 (None unless want_dh0).
    `grads` may hold preallocated outputs under the same keys.
    """
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, D)")
    batch, L, Dc = x.shape
    dev = x.device
    io = _io(x)
    dt = x.dtype
    for t, name in ((x, "x"), (delta, "delta"), (dout, "dout")):
        _need(t, name, (batch, L, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, L, Dc), dt, dev)
    _need(B, "B", (batch, L, N_STATE), dt, dev)
    _need(C, "C", (batch, L, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    for t, name in ((h0, "h0"), (dh_last, "dh_last")):
        if t is not None:
            _need(t, name, (batch, Dc, N_STATE), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(grads or {})
    shapes = {"x": ((batch, L, Dc), dt), "delta": ((batch, L, Dc), dt), "z": ((batch, L, Dc), dt),
              "B": ((batch, L, N_STATE), torch.float32), "C": ((batch, L, N_STATE), torch.float32),
              "A": ((Dc, N_STATE), torch.float32), "Dskip": ((Dc,), torch.float32),
              "dt_bias": ((Dc,), torch.float32), "h0": ((batch, Dc, N_STATE), torch.float32)}
    for k, (shape, dty) in shapes.items():
        if (k == "z" and z is None) or (k == "h0" and not want_dh0):
            g[k] = None
            continue
        if g.get(k) is None:
            g[k] = torch.empty(shape, dtype=dty, device=dev)
        _need(g[k], "grad " + k, shape, dty, dev)
    nws = bwd_workspace_bytes(batch, L, Dc, io, chunk_len)
    if workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nws:
        raise ValueError(f"workspace too small: {nws} bytes needed")
    rc = lib().ssm_scan_bwd(_ptr(x), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias),
                            _ptr(h0), _ptr(dout), _ptr(dh_last),
                            _ptr(g["x"]), _ptr(g["delta"]), _ptr(g["z"]), _ptr(g["B"]), _ptr(g["C"]),
                            _ptr(g["A"]), _ptr(g["Dskip"]), _ptr(g["dt_bias"]), _ptr(g["h0"]),
                            batch, L, Dc, N_STATE, io, chunk_len,
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)
    return {k: g[k] for k in BWD_OUTPUTS}


def state_update(h, x, delta, A, B, C, D, dt_bias, z=None, out=None):
    """One decode token: updates the float32 state h (batch, D, 16) in place, returns y (batch, D)."""
    if x.dim() != 2:
        raise ValueError("x must be (batch, D)")
    batch, Dc = x.shape
    dev = x.device
    io = _io(x)
    dt = x.dtype
    _need(h, "h", (batch, Dc, N_STATE), torch.float32, dev)
    _need(x, "x", (batch, Dc), dt, dev)
    _need(delta, "delta", (batch, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, Dc), dt, dev)
    _need(B, "B", (batch, N_STATE), dt, dev)
    _need(C, "C", (batch, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", (batch, Dc), dt, dev)
    rc = lib().ssm_state_update(_ptr(h), _ptr(x), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
                                _ptr(dt_bias), _ptr(y), batch, Dc, N_STATE, io, _stream(dev))
    _check(rc)
    return y


def conv_state_update(h, conv_state, xin, conv_w, conv_b, delta, A, B, C, D, dt_bias, z=None, out=None):
    """One decode token through the local convolution: h (batch, D, 16) and conv_state
    (batch, K-1, D) are updated in place; returns y (batch, D)."""
    if xin.dim() != 2:
        raise ValueError("xin must be (batch, D)")
    batch, Dc = xin.shape
    dev = xin.device
    io = _io(xin)
    dt = xin.dtype
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be (D, K)")
    K = conv_w.shape[1]
    _need(conv_w, "conv_w", (Dc, K), torch.float32, dev)
    _need(conv_b, "conv_b", (Dc,), torch.float32, dev)
    if K > 1:
        _need(conv_state, "conv_state", (batch, K - 1, Dc), dt, dev)
    _need(h, "h", (batch, Dc, N_STATE), torch.float32, dev)
    _need(delta, "delta", (batch, Dc), dt, dev)
    if z is not None:
        _need(z, "z", (batch, Dc), dt, dev)
    _need(B, "B", (batch, N_STATE), dt, dev)
    _need(C, "C", (batch, N_STATE), dt, dev)
    _need(A, "A", (Dc, N_STATE), torch.float32, dev)
    _need(D, "D", (Dc,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (Dc,), torch.float32, dev)
    y = torch.empty_like(xin) if out is None else out
    _need(y, "out", (batch, Dc), dt, dev)
    rc = lib().ssm_conv_state_update(_ptr(h), _ptr(conv_state if K > 1 else None), _ptr(xin), _ptr(conv_w),
                                     _ptr(conv_b), K, _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
                                     _ptr(dt_bias), _ptr(y), batch, Dc, N_STATE, io, _stream(dev))
    _check(rc)
    return y


def ssd_plan(batch: int, L: int, H: int, N: int, P: int = 64) -> Tuple[int, int]:
    """(segments per sequence, chunks of 64 tokens per segment) ssd_fwd uses for this shape."""
    ns, sc = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ssm_ssd_fwd_plan(batch, L, H, P, N, SSM_BF16, ctypes.byref(ns), ctypes.byref(sc)))
    return ns.value, sc.value


def ssd_workspace_bytes(batch: int, L: int, H: int, N: int, P: int = 64) -> int:
    """Device bytes ssd_fwd needs as workspace (the per-chunk C . B products, and the segment states when
    the sequences are cut into segments)."""
    n = lib().ssm_ssd_fwd_workspace_bytes(batch, L, H, P, N, SSM_BF16)
    if n < 0:
        _check(n)
    return n


def ssd_fwd(x, delta, A, B, C, D, dt_bias, z=None, h0=None, return_last_state: bool = True, out=None,
            workspace=None):
    """SSD (Mamba-2 style) layer with a scalar decay per head.

    x, z: (batch, L, H, 64); delta: (batch, L, H); B, C: (batch, L, N) with N
    = 64, 128 or 256, all bfloat16; A, D, dt_bias: (H,) float32; h0: (batch, H,
    64, N) float32; workspace: a device tensor of at least
    ssd_workspace_bytes(...) bytes (allocated here when None).  Returns
    (y, h_last).
    """
    if x.dim() != 4:
        raise ValueError("x must be (batch, L, H, P)")
    batch, L, H, P = x.shape
    dev = x.device
    io = _io(x)
    dt = x.dtype
    N = B.shape[-1]
    _need(x, "x", (batch, L, H, P), dt, dev)
    _need(delta, "delta", (batch, L, H), dt, dev)
    if z is not None:
        _need(z, "z", (batch, L, H, P), dt, dev)
    _need(B, "B", (batch, L, N), dt, dev)
    _need(C, "C", (batch, L, N), dt, dev)
    for t, name in ((A, "A"), (D, "D"), (dt_bias, "dt_bias")):
        _need(t, name, (H,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (batch, H, P, N), torch.float32, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", (batch, L, H, P), dt, dev)
    h_last = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev) if return_last_state else None
    if io == SSM_BF16 and N in (64, 128, 256) and P == 64:
        nws = ssd_workspace_bytes(batch, L, H, N, P)
        if workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
        elif workspace.numel() * workspace.element_size() < nws:
            raise ValueError(f"workspace too small: {nws} bytes needed")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().ssm_ssd_fwd(_ptr(x), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias),
                           _ptr(h0), _ptr(y), _ptr(h_last), batch, L, H, P, N, io, _ptr(workspace), nbytes,
                           _stream(dev))
    _check(rc)
    return y, h_last


def timing_enable(on: bool = True, kernel: Optional[str] = None) -> None:
    """Bracket later launches of `kernel` (every kernel if None) with HIP events on their stream."""
    _check(lib().ssm_timing_enable(1 if on else 0, kernel.encode() if (on and kernel) else None))


def timing_collect(max_kernels: int = 16) -> dict:
    """{kernel name: (launches, total ms)} recorded since the last collect (waits for the events)."""
    names = (ctypes.c_char_p * max_kernels)()
    cnt = (ctypes.c_int64 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = lib().ssm_timing_collect(max_kernels, names, cnt, ms)
    if n < 0:
        _check(n)
    return {names[i].decode(): (int(cnt[i]), float(ms[i])) for i in range(min(n, max_kernels))}
