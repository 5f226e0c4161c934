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

Backward.  scan_bwd returns the gradient of J = sum(dout * out) +
sum(dh_last * h_L) with respect to every input: the chain rule of the
recurrence above, run backward in time over the stored float64 states.
Training differentiates through the scan and the pages' own kernel recomputes
the states for it instead of storing them ("DL0170 ...", point (3) and the
paragraph after Figure 1); here they are simply stored.

Local convolution.  conv_silu is the block's short local mixing step before
the scan ("Mamba", "Block Structure": a local convolution adds short-range
context; "Mamba: State Space Models", "What a Mamba Block Contains": a short
convolution for local mixing).  The pages give neither its width nor an
activation; the reading taken here is a causal depthwise convolution along
time of width K <= 4 with a per-channel bias, followed by silu:
x_t = silu(b_d + sum_k w_dk * xin_{t-K+1+k}), with the K-1 inputs before the
sequence taken from conv_init (zeros when None).  conv_scan_fwd feeds its
output to scan_fwd as x.

Parity status: pinned.  The test suite checks this module against the
Delta -> 0 pass-through, the LTI convolution (direct sum, FFT and geometric
closed form), a brute-force causal-matrix sum ("Mamba", "Relation to
Mamba-2"), the overwrite limit ("DL0170 ...", point (2)), pure decay in
closed form, sequence splitting and chained decode steps, and linearity; the
backward against central finite differences of that brute-force sum, exact
dot-product identities of the inputs in which the output is linear, the LTI
transposed convolution, a one-token closed form and gradient splitting; the
local convolution against numpy.convolve, scipy.signal.lfilter, impulse
responses, causality and stream splitting through conv_init.
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


# ---------------------------------------------------------------------------
# the backward pass
# ---------------------------------------------------------------------------

def _sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def scan_bwd(x, delta, A, B, C, Dskip, dt_bias, dout, z=None, h0=None, dh_last=None, io: str = "f64"):
    """Gradients of J = sum(dout * out) + sum(dh_last * h_L) for scan_fwd.

    Same inputs as scan_fwd, plus dout (bt, L, D) (stored like x) and dh_last
    (bt, D, N) or None (zero; always numbers, not io storage).  Returns a dict
    of float64 arrays keyed by input name: x, delta, z (None when ungated), A,
    B, C, Dskip, dt_bias, h0 (the gradient with respect to the starting state,
    also when h0 itself is None, i.e. zeros).

    Forward (stored): Delta_t = softplus(v_t), v_t = delta_t + dt_bias;
    Abar_t = exp(Delta_t A); h_t = Abar_t h_{t-1} + Delta_t x_t B_t;
    y_t = C_t . h_t + Dskip x_t; out_t = y_t silu(z_t).
    Backward: dy_t = dout_t silu(z_t); mu_t = dJ/dh_t obeys
    mu_t = C_t dy_t + Abar_{t+1} mu_{t+1}, with mu_{L-1} also receiving
    dh_last; every other gradient is a product of mu_t with the forward
    quantities of the same token.
    """
    if io != "f64":
        x, delta, B, C, dout = (decode(a, io) for a in (x, delta, B, C, dout))
        z = None if z is None else decode(z, io)
    x = np.asarray(x, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    Dskip = np.asarray(Dskip, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    bt, L, D = x.shape
    N = A.shape[1]
    v = np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    Delta = softplus(v)

    # forward, keeping every state: hs[:, t + 1] = h_t, hs[:, 0] = h0
    hs = np.empty((bt, L + 1, D, N))
    hs[:, 0] = 0.0 if h0 is None else np.asarray(h0, dtype=np.float64)
    for t in range(L):
        Abar = np.exp(Delta[:, t, :, None] * A[None, :, :])
        hs[:, t + 1] = Abar * hs[:, t] + (Delta[:, t, :] * x[:, t, :])[:, :, None] * B[:, t, None, :]
    y = np.einsum("btdn,btn->btd", hs[:, 1:], C) + Dskip[None, None, :] * x

    if z is not None:
        z = np.asarray(z, dtype=np.float64)
        sg = _sigmoid(z)
        dy = dout * z * sg
        dz = dout * y * sg * (1.0 + z * (1.0 - sg))   # d silu / dz = sigmoid (1 + z (1 - sigmoid))
    else:
        dy = dout
        dz = None

    dx = np.empty((bt, L, D))
    dDelta = np.empty((bt, L, D))
    dB = np.empty((bt, L, N))
    dC = np.einsum("btd,btdn->btn", dy, hs[:, 1:])
    dA = np.zeros((D, N))
    # carried adjoint: the part of mu_t that comes from later tokens (and dh_last)
    carry = np.zeros((bt, D, N)) if dh_last is None else np.array(dh_last, dtype=np.float64)
    for t in range(L - 1, -1, -1):
        mu = dy[:, t, :, None] * C[:, t, None, :] + carry                 # (bt, D, N)
        Abar = np.exp(Delta[:, t, :, None] * A[None, :, :])
        w = mu * Abar * hs[:, t]                                          # dJ/d(Delta_t A) per state
        du = np.einsum("bdn,bn->bd", mu, B[:, t])                         # dJ/d(Delta_t x_t)
        dx[:, t] = du * Delta[:, t] + dy[:, t] * Dskip[None, :]
        dDelta[:, t] = du * x[:, t] + np.einsum("bdn,dn->bd", w, A)
        dB[:, t] = np.einsum("bdn,bd->bn", mu, Delta[:, t] * x[:, t])
        dA += np.einsum("bdn,bd->dn", w, Delta[:, t])
        carry = Abar * mu
    dv = dDelta * _sigmoid(v)                                             # softplus' = sigmoid
    return dict(x=dx, delta=dv, z=dz, A=dA, B=dB, C=dC,
                Dskip=np.einsum("btd,btd->d", dy, x), dt_bias=dv.sum(axis=(0, 1)), h0=carry)


# ---------------------------------------------------------------------------
# the local convolution before the scan
# ---------------------------------------------------------------------------

def conv_silu(xin, w, b, conv_init=None, io: str = "f64"):
    """silu of a causal depthwise convolution along time.

    xin: (bt, L, D); w: (D, K) float32, tap k weighting xin_{t-K+1+k};
    b: (D,); conv_init: (bt, K-1, D) inputs before the sequence, or None
    (zeros), stored like xin.  Returns x (bt, L, D) float64.
    """
    if io != "f64":
        xin = decode(xin, io)
        conv_init = None if conv_init is None else decode(conv_init, io)
    xin = np.asarray(xin, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bt, L, D = xin.shape
    K = w.shape[1]
    head = np.zeros((bt, K - 1, D)) if conv_init is None else np.asarray(conv_init, dtype=np.float64)
    padded = np.concatenate([head, xin], axis=1)                       # (bt, K-1+L, D)
    v = np.broadcast_to(b, (bt, L, D)).copy()
    for t in range(L):
        for k in range(K):
            v[:, t, :] += w[None, :, k] * padded[:, t + k, :]
    return silu(v)


def conv_scan_fwd(xin, conv_w, conv_b, delta, A, B, C, Dskip, dt_bias, z=None, h0=None, conv_init=None,
                  io: str = "f64"):
    """The scan fed by the local convolution: scan_fwd(conv_silu(xin), ...)."""
    x = conv_silu(xin, conv_w, conv_b, conv_init, io=io)
    if io != "f64":
        delta, B, C = (decode(a, io) for a in (delta, B, C))
        z = None if z is None else decode(z, io)
    return scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=h0)


def conv_state_update(conv_state, h, xin, conv_w, conv_b, delta, A, B, C, Dskip, dt_bias, z=None,
                      io: str = "f64"):
    """One decode token through the local convolution and the scan.

    conv_state: (bt, K-1, D) the last K-1 inputs (stored like xin); h: (bt, D, N);
    xin, delta, z: (bt, D); B, C: (bt, N).  Returns (out (bt, D), h_new,
    conv_state_new) where conv_state_new is [conv_state, xin] without its
    oldest row; the inputs are not modified.
    """
    as_seq = lambda a: None if a is None else np.asarray(a)[:, None, :]
    y, hn = conv_scan_fwd(as_seq(xin), conv_w, conv_b, as_seq(delta), A, as_seq(B), as_seq(C), Dskip, dt_bias,
                          z=as_seq(z), h0=h, conv_init=conv_state, io=io)
    both = np.concatenate([np.asarray(conv_state), np.asarray(xin)[:, None, :]], axis=1)
    return y[:, 0, :], hn, both[:, 1:]
