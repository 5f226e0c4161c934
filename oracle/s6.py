"""Float64 CPU oracle for the selective scan (S6) and its single-token decode step.

TEST INFRASTRUCTURE ONLY. This module is the slow, plainly written definition
that the HIP library is checked against. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the library never does,
and the two share no code (the oracle decodes its own bfloat16 inputs and
computes everything in float64 with NumPy).

What it computes, for every batch row b, channel d and state index n
(pages cited by title and section):

* Step size.  Delta_t = softplus(delta_t + dt_bias_d).  The pages make the step
  size a function of the current token ("Mamba: State Space Models", "The Key
  Innovation: Selectivity") and note that its initialisation puts it at a
  sensible time scale ("DL0170 Mamba Selective SSM vs Attention",
  "Mathematical Formulation"); they do not print the map itself. The softplus of a token
  projection plus a per-channel bias is the reading taken here; the
  projection delta_t arrives as an input.
* Discretisation.  Abar_t = exp(Delta_t * A_dn): zero-order hold of the
  diagonal A ("DL0170 ...", "Mathematical Formulation"; "Mamba &
  State-Space Sequence Models", "Core mechanics").  For the input term the
  DL0170 page has Mamba drop the exact zero-order-hold input matrix for the
  first-order Bbar_t = Delta_t * B_t, which is what is used here.
* Recurrence.  h_t = Abar_t * h_{t-1} + Bbar_t * x_t, starting from h_0
  ("Mamba", "Scan View" and "Main Claim"; "Mamba Selective State-Space
  Module", "Math Or Compute Schema").  h_0 is zero unless given.
* Readout.  y_t = sum_n C_tn * h_tn + Dskip_d * x_t, reading the state *after*
  the token's update, as y_t = C_t h_t on every page.  The skip term is not on
  the pages; it is part of the S6 layer this library implements.
* Gate.  out_t = y_t * silu(z_t) when a gate z is given ("Mamba",
  "Selectivity" and "Block Structure" put a gate on the block's output; no
  page names its function, silu is the reading taken), else out_t = y_t.

B and C are (batch, L, N) and shared by all channels of a batch row.

Parity status: pinned.  The test suite checks this module against the
Delta -> 0 pass-through, the LTI convolution (direct sum, FFT and geometric
closed form), a brute-force causal-matrix sum ("Mamba", "Relation to
Mamba-2"), the overwrite limit ("DL0170 ...", point (2)), pure decay in
closed form, sequence splitting and chained decode steps, and linearity.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# input decoding (the oracle's own; exact)
# ---------------------------------------------------------------------------

def decode(a, io: str) -> np.ndarray:
    """Inputs as float64: bfloat16 bit patterns (uint16) or float32 values."""
    a = np.asarray(a)
    if io == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are carried as uint16 bit patterns")
        wide = a.astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
            return wide.view(np.float32).astype(np.float64)
    if io == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 inputs must be float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown io dtype {io!r}")


# ---------------------------------------------------------------------------
# elementwise maps
# ---------------------------------------------------------------------------

def softplus(v):
    """log(1 + e^v), evaluated without overflow."""
    return np.logaddexp(0.0, v)


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# the scan
# ---------------------------------------------------------------------------

def recurrence(Delta, x, A, B, C, Dskip, h0=None):
    """The selective recurrence and readout, given the step sizes directly.

    Delta, x: (bt, L, D); A: (D, N); B, C: (bt, L, N); Dskip: (D,);
    h0: (bt, D, N) or None (zeros).  All float64.  Returns the ungated y
    (bt, L, D) and the final state h_L (bt, D, N).
    """
    Delta = np.asarray(Delta, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    Dskip = np.asarray(Dskip, dtype=np.float64)
    bt, L, D = x.shape
    N = A.shape[1]
    h = np.zeros((bt, D, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((bt, L, D))
    for t in range(L):
        Abar = np.exp(Delta[:, t, :, None] * A[None, :, :])           # (bt, D, N)
        Bbar_x = (Delta[:, t, :] * x[:, t, :])[:, :, None] * B[:, t, None, :]
        h = Abar * h + Bbar_x
        y[:, t, :] = np.einsum("bdn,bn->bd", h, C[:, t, :]) + Dskip[None, :] * x[:, t, :]
    return y, h


def scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=None, h0=None, io: str = "f64"):
    """Whole-sequence selective scan.

    x, delta, z: (bt, L, D); B, C: (bt, L, N); A: (D, N); Dskip, dt_bias: (D,);
    h0: (bt, D, N) or None.  With io="bf16" or "f32" the sequence inputs are
    decoded from that storage first; with io="f64" they are taken as numbers.
    Returns (out, h_L) in float64.
    """
    if io != "f64":
        x, delta, B, C = (decode(a, io) for a in (x, delta, B, C))
        z = None if z is None else decode(z, io)
    v = np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    Delta = softplus(v)
    y, h = recurrence(Delta, x, A, B, C, Dskip, h0)
    if z is not None:
        y = y * silu(z)
    return y, h


def state_update(h, x, delta, A, B, C, Dskip, dt_bias, z=None, io: str = "f64"):
    """One decode token against a cached state: the scan with L = 1.

    h: (bt, D, N) state before the token; x, delta, z: (bt, D); B, C: (bt, N).
    Returns (out (bt, D), h_new (bt, D, N)); the input h is not modified.
    """
    if io != "f64":
        x, delta, B, C = (decode(a, io) for a in (x, delta, B, C))
        z = None if z is None else decode(z, io)
    x = np.asarray(x, dtype=np.float64)[:, None, :]
    delta = np.asarray(delta, dtype=np.float64)[:, None, :]
    B = np.asarray(B, dtype=np.float64)[:, None, :]
    C = np.asarray(C, dtype=np.float64)[:, None, :]
    zz = None if z is None else np.asarray(z, dtype=np.float64)[:, None, :]
    y, hn = scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=zz, h0=h)
    return y[:, 0, :], hn
