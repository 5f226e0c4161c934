"""Pins for the float64 SSD oracle (oracle/ssd.py): results that do not come from it.

Each pin takes the oracle module ``m`` (exposing ssd_fwd) and raises
AssertionError on a disagreement; tests/test_ssd_oracle.py also runs them on
copies with planted mistakes.  Pages are cited by title and section.
"""
from __future__ import annotations

import numpy as np

import oracle.s6 as s6
from oracle_pins import _close, _sp


def _rng(seed):
    return np.random.default_rng([392, seed])


def ssd_case(seed, bt=2, L=30, H=3, P=4, N=8, gated=True, with_h0=True):
    r = _rng(seed)
    return dict(x=r.standard_normal((bt, L, H, P)), delta=r.standard_normal((bt, L, H)),
                A=-np.exp(r.uniform(-1.0, 1.0, size=H)), B=r.standard_normal((bt, L, N)),
                C=r.standard_normal((bt, L, N)), Dskip=r.uniform(0.5, 1.5, size=H),
                dt_bias=r.uniform(-3.0, 0.0, size=H),
                z=r.standard_normal((bt, L, H, P)) if gated else None,
                h0=r.standard_normal((bt, H, P, N)) if with_h0 else None)


def _run(m, c, sl=slice(None), h0="case"):
    return m.ssd_fwd(c["x"][:, sl], c["delta"][:, sl], c["A"], c["B"][:, sl], c["C"][:, sl], c["Dskip"],
                     c["dt_bias"], z=None if c["z"] is None else c["z"][:, sl],
                     h0=c["h0"] if isinstance(h0, str) else h0)


def pin_ssd_equals_s6_per_head(m):
    """Each head is an S6 scan of its P channels with A_dn = A_h for every state n and the
    head's step size on every channel (the pinned S6 oracle, oracle/s6.py)."""
    for gated in (True, False):
        c = ssd_case(1, gated=gated)
        y, h = _run(m, c)
        bt, L, H, P = c["x"].shape
        N = c["B"].shape[-1]
        for hd in range(H):
            A6 = np.full((P, N), c["A"][hd])
            d6 = np.repeat(c["delta"][:, :, hd:hd + 1], P, axis=2)
            y6, h6 = s6.scan_fwd(c["x"][:, :, hd], d6, A6, c["B"], c["C"], np.full(P, c["Dskip"][hd]),
                                 np.full(P, c["dt_bias"][hd]), z=None if c["z"] is None else c["z"][:, :, hd],
                                 h0=c["h0"][:, hd])
            _close(y[:, :, hd], y6, 1e-13, f"head {hd} y (gated={gated})")
            _close(h[:, hd], h6, 1e-13, f"head {hd} h_L")


def pin_ssd_matrix_mixer(m):
    """y_t = sum_{i<=t} (C_t . B_i) exp(A sum_{i<j<=t} Delta_j) Delta_i x_i + D x_t
    + C_t . exp(A sum_{j<=t} Delta_j) h0 ("Mamba", "Relation to Mamba-2"), summed explicitly."""
    c = ssd_case(2, L=17, gated=False)
    y, h = _run(m, c)
    bt, L, H, P = c["x"].shape
    Delta = _sp(c["delta"] + c["dt_bias"][None, None, :])
    ref = np.zeros_like(y)
    for b in range(bt):
        for hd in range(H):
            for t in range(L):
                acc = c["Dskip"][hd] * c["x"][b, t, hd]
                for i in range(t + 1):
                    decay = np.exp(c["A"][hd] * Delta[b, i + 1:t + 1, hd].sum())
                    acc = acc + (c["C"][b, t] @ c["B"][b, i]) * decay * Delta[b, i, hd] * c["x"][b, i, hd]
                acc = acc + np.exp(c["A"][hd] * Delta[b, :t + 1, hd].sum()) * (c["h0"][b, hd] @ c["C"][b, t])
                ref[b, t, hd] = acc
    _close(y, ref, 1e-12, "matrix mixer")


def pin_ssd_split(m):
    """ssd(0:L) = ssd(L1:L, h0 = h_L1) after ssd(0:L1)."""
    c = ssd_case(3)
    full, hf = _run(m, c)
    for L1 in (1, 12, 29):
        a, ha = _run(m, c, slice(0, L1))
        b, hb = _run(m, c, slice(L1, None), h0=ha)
        _close(np.concatenate([a, b], axis=1), full, 1e-13, f"split {L1}")
        _close(hb, hf, 1e-13, f"split state {L1}")


SSD_PINS = [pin_ssd_equals_s6_per_head, pin_ssd_matrix_mixer, pin_ssd_split]
