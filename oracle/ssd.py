"""Float64 CPU oracle for the SSD (Mamba-2 style) layer.

TEST INFRASTRUCTURE ONLY, like oracle/s6.py: the slow, plainly written
definition the HIP library is checked against; only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it, and it shares no
code with the library.

What it computes (pages cited by title and section).  "Mamba", "Relation to
Mamba-2" writes the selective SSM as a causal matrix mixer,
y_t = sum_{i<=t} C_t (prod_{j=i+1..t} A_j) B_i x_i, and credits Mamba-2 with a
faster block/chunk algorithm for it; "Mamba & State-Space Sequence Models",
"Core mechanics" calls this a duality between structured SSMs and a class of
linear attention; "DL0170 Mamba Selective SSM vs Attention" (paragraph after
Figure 1) has Mamba-2 raise the state size N from 16 up to 256.  The pages do
not print the layer itself.  The reading taken here (the structure under
which the matrix mixer is an attention-like masked product):

* heads h = 0..H-1, each with P channels; the per-head transition is a
  scalar times the identity: Abar_t,h = exp(Delta_t,h * A_h), A_h < 0;
* Delta_t,h = softplus(delta_t,h + dt_bias_h), one step size per head;
* B_t, C_t (length N) shared by all heads of a batch row;
* state h_t,h (P x N) = Abar_t,h h_{t-1,h} + Delta_t,h x_t,h B_t^T;
* y_t,h = h_t,h C_t + Dskip_h x_t,h (readout after the update, as in S6),
  out = y * silu(z) when a gate z is given.

Layouts: x, z, y (bt, L, H, P); delta (bt, L, H); B, C (bt, L, N); A, Dskip,
dt_bias (H,); h0, h_L (bt, H, P, N).

Parity status: pinned.  The tests check this module against the S6 oracle
(each head is an S6 scan over its P channels whose N states all share the
head's decay), the explicit causal matrix-mixer sum, sequence splitting, and a
float64 chunked evaluation (intra-chunk masked products plus carried states).
"""
from __future__ import annotations

import numpy as np

from .s6 import decode, silu, softplus


def ssd_fwd(x, delta, A, B, C, Dskip, dt_bias, z=None, h0=None, io: str = "f64"):
    """Whole-sequence SSD layer.  Returns (out (bt, L, H, P), h_L (bt, H, P, N)) in float64."""
    if io != "f64":
        x, delta, B, C = (decode(a, io) for a in (x, delta, B, C))
        z = None if z is None else decode(z, io)
    x = np.asarray(x, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    Dskip = np.asarray(Dskip, dtype=np.float64)
    bt, L, H, P = x.shape
    N = B.shape[-1]
    Delta = softplus(np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, None, :])
    h = np.zeros((bt, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((bt, L, H, P))
    for t in range(L):
        decay = np.exp(Delta[:, t] * A[None, :])                               # (bt, H)
        inp = (Delta[:, t, :, None] * x[:, t])[..., None] * B[:, t, None, None, :]  # (bt, H, P, N)
        h = decay[:, :, None, None] * h + inp
        y[:, t] = np.einsum("bhpn,bn->bhp", h, C[:, t]) + Dskip[None, :, None] * x[:, t]
    if z is not None:
        y = y * silu(z)
    return y, h
