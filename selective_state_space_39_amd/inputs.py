"""Seeded synthetic inputs for the selective scan (S6).

This module only draws random numbers and lays them out. It evaluates none of
the scan's arithmetic (no discretisation, recurrence, readout or gate), so the
float64 oracle and the HIP path can both be fed from it without sharing any of
the method's code.

Two small pieces of arithmetic do live here, and both are input *placement*,
not the method:

* ``bf16_encode`` rounds float32 values to bfloat16 bit patterns
  (round-to-nearest-even). Both sides then consume the same 16-bit patterns.
* ``inv_softplus`` places a desired step size: the recipes state dt_bias, and
  the long-context Δ blocks, as the value whose softplus is a chosen Δ.

Layouts (all C-contiguous, row-major):

* x, delta, z: (batch, L, D), D fastest.
* B, C: (batch, L, N), shared by all D channels of a batch row.
* A: (D, N) float32; Dskip, dt_bias: (D,) float32.
* h0 / decode state: (batch, D, N) float32, N fastest.

bf16 tensors are carried as ``numpy.uint16`` bit patterns; fp32 tensors as
``numpy.float32``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

N_STATE = 16
SEED_ROOT = 39

# Named whole-sequence workloads and the seed each is drawn from. Sizes follow
# the S6 layer shapes they are named after; the "D" here is the already-expanded
# inner width (two times the model width).
SCAN_WORKLOADS = {
    "tiny-f32": dict(batch=1, L=256, D=16, io="f32", delta="normal", delta_sigma=0.5, seed=(SEED_ROOT, 1)),
    "mamba-130m-layer": dict(batch=8, L=2048, D=1536, io="bf16", delta="normal", delta_sigma=0.5,
                             seed=(SEED_ROOT, 2)),
    "mamba-2.8b-layer": dict(batch=4, L=2048, D=5120, io="bf16", delta="normal", delta_sigma=1.0,
                             seed=(SEED_ROOT, 3)),
    "long-context-128k": dict(batch=1, L=131072, D=2048, io="bf16", delta="blocks", block=64,
                              seed=(SEED_ROOT, 4)),
}
# Chained single-token decode against a cached state: (batch, D), 1000 steps,
# drawn from decode_params / decode_token.
DECODE_WORKLOAD = dict(name="decode-256x5120", batch=256, D=5120, io="bf16", steps=1000, seed=(SEED_ROOT, 5))


# ----------------------------------------------------------------------------
# bfloat16 bit patterns
# ----------------------------------------------------------------------------

def bf16_encode(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    NaN maps to a quiet NaN; infinities and overflow to +-inf follow from the
    rounding itself.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    out = np.empty(f.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24  # bound the uint32 temporaries on huge tensors
    for s in range(0, flat_u.size, step):
        blk = flat_u[s:s + step]
        lsb = (blk >> np.uint32(16)) & np.uint32(1)
        r = ((blk + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
        nan = (blk & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = ((blk[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
        flat_o[s:s + step] = r
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def inv_softplus(u: np.ndarray) -> np.ndarray:
    """The v with log(1 + e^v) = u, for u > 0, in float64 (= u + log(1 - e^-u))."""
    u = np.asarray(u, dtype=np.float64)
    return u + np.log(-np.expm1(-u))


# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------

@dataclass
class ScanInputs:
    io: str                      # "f32" or "bf16": dtype of x, delta, z, B, C and y
    x: np.ndarray
    delta: np.ndarray
    z: Optional[np.ndarray]
    B: np.ndarray
    C: np.ndarray
    A: np.ndarray                # (D, N) float32
    Dskip: np.ndarray            # (D,) float32
    dt_bias: np.ndarray          # (D,) float32
    h0: Optional[np.ndarray] = None   # (batch, D, N) float32
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        b, L, D = self.x.shape
        return b, L, D, self.B.shape[-1]


@dataclass
class DecodeToken:
    io: str
    x: np.ndarray                # (batch, D)
    delta: np.ndarray            # (batch, D)
    z: Optional[np.ndarray]      # (batch, D)
    B: np.ndarray                # (batch, N)
    C: np.ndarray                # (batch, N)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------

def _as_io(a32: np.ndarray, io: str) -> np.ndarray:
    if io == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if io == "bf16":
        return bf16_encode(a32)
    raise ValueError(f"unknown io dtype {io!r}")


def channel_params(rng: np.random.Generator, D: int, N: int = N_STATE):
    """A, Dskip, dt_bias for D channels.

    A_dn = -(n+1) (the S4D-real initialisation), Dskip = 1, and dt_bias is the
    inverse softplus of a step u drawn log-uniformly in [1e-3, 0.1].
    """
    u = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=D))
    dt_bias = inv_softplus(u).astype(np.float32)
    A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    Dskip = np.ones(D, dtype=np.float32)
    return A, Dskip, dt_bias


def _normal(rng, shape, sigma=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def block_delta(rng, batch, L, D, dt_bias, block=64, lo=1e-3, hi=1.0, jitter=0.1):
    """delta whose step size alternates every ``block`` tokens.

    Even blocks (the first included) target a step near ``lo`` (the state is
    carried through almost unchanged); odd blocks target a step near ``hi``
    (the state is mostly overwritten). Per (t, d) the target is
    c * exp(jitter * eps), eps ~ N(0, 1); delta is the inverse softplus of the
    target minus dt_bias_d. Returned in float32 (rounding to the io dtype
    happens afterwards, so the realised step is what the rounded delta gives).
    """
    eps = rng.standard_normal(size=(batch, L, D), dtype=np.float32)
    out = np.empty((batch, L, D), dtype=np.float32)
    level = np.where((np.arange(L) // block) % 2 == 0, lo, hi)
    bias = dt_bias.astype(np.float64)
    tstep = max(1, (1 << 22) // max(1, D))
    for b in range(batch):
        for t0 in range(0, L, tstep):
            t1 = min(L, t0 + tstep)
            target = level[t0:t1, None] * np.exp(jitter * eps[b, t0:t1].astype(np.float64))
            out[b, t0:t1] = (inv_softplus(target) - bias[None, :]).astype(np.float32)
    return out


def make_scan_inputs(batch: int, L: int, D: int, N: int = N_STATE, io: str = "bf16",
                     seed=(SEED_ROOT, 0), delta: str = "normal", delta_sigma: float = 0.5,
                     block: int = 64, gated: bool = True, with_h0: bool = False,
                     A_random: bool = False) -> ScanInputs:
    """Seeded inputs for one whole-sequence scan.

    Draw order from ``numpy.random.default_rng(seed)``: u (-> dt_bias), x,
    delta (or the block-jitter eps), z, B, C, h0. x, z, B, C ~ N(0, 1);
    delta ~ N(0, delta_sigma^2) or the alternating blocks; h0 ~ N(0, 1).
    With ``A_random`` the S4D-real A is replaced by A_dn = -exp(U(-1.5, 1.5)),
    different for every channel and state, drawn from the stream (*seed, 2).
    """
    rng = np.random.default_rng(list(seed) if not isinstance(seed, int) else seed)
    A, Dskip, dt_bias = channel_params(rng, D, N)
    x = _normal(rng, (batch, L, D))
    if delta == "normal":
        dl = _normal(rng, (batch, L, D), delta_sigma)
    elif delta == "blocks":
        dl = block_delta(rng, batch, L, D, dt_bias, block=block)
    else:
        raise ValueError(delta)
    z = _normal(rng, (batch, L, D)) if gated else None
    B = _normal(rng, (batch, L, N))
    C = _normal(rng, (batch, L, N))
    h0 = _normal(rng, (batch, D, N)) if with_h0 else None
    if A_random:
        ra = np.random.default_rng(list(seed) + [2] if not isinstance(seed, int) else [seed, 2])
        A = (-np.exp(ra.uniform(-1.5, 1.5, size=(D, N)))).astype(np.float32)
    return ScanInputs(io=io, x=_as_io(x, io), delta=_as_io(dl, io),
                      z=None if z is None else _as_io(z, io),
                      B=_as_io(B, io), C=_as_io(C, io), A=A, Dskip=Dskip, dt_bias=dt_bias,
                      h0=h0, meta=dict(seed=seed, delta=delta))


@dataclass
class GradOutputs:
    io: str
    dout: np.ndarray                  # (batch, L, D) io storage: gradient of the scan output
    dh_last: Optional[np.ndarray]     # (batch, D, N) float32: gradient of the final state, or None


def make_grad_outputs(batch: int, L: int, D: int, N: int = N_STATE, io: str = "bf16", seed=(SEED_ROOT, 0),
                      with_dh_last: bool = True) -> GradOutputs:
    """Upstream gradients for a backward pass, from the stream (*seed, 1).

    Draw order: dout ~ N(0, 1) (rounded to the io dtype), dh_last ~ N(0, 1).
    """
    rng = np.random.default_rng(list(seed) + [1] if not isinstance(seed, int) else [seed, 1])
    dout = _normal(rng, (batch, L, D))
    dh = _normal(rng, (batch, D, N)) if with_dh_last else None
    return GradOutputs(io=io, dout=_as_io(dout, io), dh_last=dh)


@dataclass
class ConvParams:
    w: np.ndarray                     # (D, K) float32, tap k weighting xin_{t-K+1+k}
    b: np.ndarray                     # (D,) float32
    init: Optional[np.ndarray]        # (batch, K-1, D) io storage: inputs before the sequence, or None


def make_conv_params(batch: int, D: int, K: int = 4, io: str = "bf16", seed=(SEED_ROOT, 0),
                     with_init: bool = False) -> ConvParams:
    """Local-convolution parameters from the stream (*seed, 3).

    Draw order: w ~ U(-1/sqrt(K), 1/sqrt(K)) (D, K), b ~ N(0, 0.1^2) (D,),
    init ~ N(0, 1) (batch, K-1, D) rounded to the io dtype.
    """
    rng = np.random.default_rng(list(seed) + [3] if not isinstance(seed, int) else [seed, 3])
    lim = 1.0 / np.sqrt(K)
    w = rng.uniform(-lim, lim, size=(D, K)).astype(np.float32)
    b = _normal(rng, (D,), 0.1)
    init = _as_io(_normal(rng, (batch, K - 1, D)), io) if (with_init and K > 1) else None
    return ConvParams(w=w, b=b, init=init)


@dataclass
class SsdInputs:
    io: str
    x: np.ndarray                 # (batch, L, H, P) io storage
    delta: np.ndarray             # (batch, L, H) io storage
    z: Optional[np.ndarray]       # (batch, L, H, P) io storage
    B: np.ndarray                 # (batch, L, N) io storage, shared by all heads
    C: np.ndarray                 # (batch, L, N) io storage
    A: np.ndarray                 # (H,) float32, negative
    Dskip: np.ndarray             # (H,) float32
    dt_bias: np.ndarray           # (H,) float32
    h0: Optional[np.ndarray] = None   # (batch, H, P, N) float32

    @property
    def shape(self):
        b, L, H, P = self.x.shape
        return b, L, H, P, self.B.shape[-1]


SSD_WORKLOAD = dict(name="mamba2-2.7b-layer", batch=8, L=2048, H=80, P=64, N=128, io="bf16", seed=(SEED_ROOT, 6))
# The same layer at the two other state sizes the kernels are built for.
SSD_WORKLOADS = {w["name"]: w for w in (
    SSD_WORKLOAD,
    dict(SSD_WORKLOAD, name="mamba2-2.7b-layer-n64", N=64, seed=(SEED_ROOT, 10)),
    dict(SSD_WORKLOAD, name="mamba2-2.7b-layer-n256", N=256, seed=(SEED_ROOT, 11)),
    # one long sequence: too few (batch row, head) sequences to fill the GPU, so they are cut into segments
    dict(SSD_WORKLOAD, name="mamba2-long-context-128k", batch=1, L=131072, seed=(SEED_ROOT, 12)))}


def make_ssd_inputs(batch: int, L: int, H: int, P: int = 64, N: int = 128, io: str = "bf16",
                    seed=(SEED_ROOT, 6), gated: bool = True, with_h0: bool = False,
                    delta_sigma: float = 0.5) -> SsdInputs:
    """Seeded inputs for the SSD layer.

    Draw order from ``numpy.random.default_rng(seed)``: A_h = -U(1, 16), u (->
    dt_bias = softplus^-1 of a log-uniform step in [1e-3, 0.1]), x, delta, z,
    B, C, h0.  x, z, B, C, h0 ~ N(0, 1); delta ~ N(0, delta_sigma^2); Dskip = 1.
    """
    rng = np.random.default_rng(list(seed) if not isinstance(seed, int) else seed)
    A = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    u = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=H))
    dt_bias = inv_softplus(u).astype(np.float32)
    x = _normal(rng, (batch, L, H, P))
    dl = _normal(rng, (batch, L, H), delta_sigma)
    z = _normal(rng, (batch, L, H, P)) if gated else None
    B = _normal(rng, (batch, L, N))
    C = _normal(rng, (batch, L, N))
    h0 = _normal(rng, (batch, H, P, N)) if with_h0 else None
    return SsdInputs(io=io, x=_as_io(x, io), delta=_as_io(dl, io), z=None if z is None else _as_io(z, io),
                     B=_as_io(B, io), C=_as_io(C, io), A=A, Dskip=np.ones(H, dtype=np.float32), dt_bias=dt_bias,
                     h0=h0)


def make_workload(name: str) -> ScanInputs:
    """The named whole-sequence workload (SCAN_WORKLOADS), seeded as listed there."""
    c = SCAN_WORKLOADS[name]
    return make_scan_inputs(c["batch"], c["L"], c["D"], N_STATE, c["io"], seed=c["seed"],
                            delta=c["delta"], delta_sigma=c.get("delta_sigma", 0.5),
                            block=c.get("block", 64))


def decode_params(batch: int = 256, D: int = 5120, N: int = N_STATE, seed=(SEED_ROOT, 5), A_random: bool = False):
    """Channel parameters and the fp32 initial cached state for a decode run.

    Draw order: u (-> dt_bias), then h0 ~ N(0, 1) of shape (batch, D, N).
    With ``A_random`` A is drawn as in ``make_scan_inputs`` (stream (*seed, 2)).
    """
    rng = np.random.default_rng(list(seed))
    A, Dskip, dt_bias = channel_params(rng, D, N)
    h0 = _normal(rng, (batch, D, N))
    if A_random:
        A = (-np.exp(np.random.default_rng(list(seed) + [2]).uniform(-1.5, 1.5, size=(D, N)))).astype(np.float32)
    return A, Dskip, dt_bias, h0


def decode_token(step: int, batch: int = 256, D: int = 5120, N: int = N_STATE, io: str = "bf16",
                 delta_sigma: float = 0.5, gated: bool = True, seed_root=(SEED_ROOT, 5)) -> DecodeToken:
    """One decode token for every sequence, seeded with (*seed_root, step).

    Draw order: x, delta, z, B, C; distributions as for the scans.
    """
    rng = np.random.default_rng(list(seed_root) + [int(step)])
    x = _normal(rng, (batch, D))
    dl = _normal(rng, (batch, D), delta_sigma)
    z = _normal(rng, (batch, D)) if gated else None
    B = _normal(rng, (batch, N))
    C = _normal(rng, (batch, N))
    return DecodeToken(io=io, x=_as_io(x, io), delta=_as_io(dl, io),
                       z=None if z is None else _as_io(z, io), B=_as_io(B, io), C=_as_io(C, io))
