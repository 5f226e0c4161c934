"""The chunk-carry algebra the long-sequence kernels rely on, checked in float64.

A chunk of tokens acts on the state as h -> exp(A * S) * h + H, where S is the
chunk's summed step size (per channel) and H is the state the chunk reaches
from zero. Composition of two such maps is
(S1, H1) then (S2, H2) = (S1 + S2, exp(A * S2) * H1 + H2), which is
associative; this is the associative structure under which "Mamba", "Scan
View" says the recurrence can be evaluated as a parallel scan. These tests
evaluate a scan chunk by chunk with that operator and compare it with the
oracle, independently of any GPU code.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


def combine(A, c1, c2):
    S1, H1 = c1
    S2, H2 = c2
    return S1 + S2, np.exp(A * S2[..., None]) * H1 + H2


def chunk_carry(Delta, x, A, B):
    """(S, H) of a chunk: summed step and the state reached from zero (float64)."""
    bt, L, D = x.shape
    h = np.zeros((bt, D, A.shape[1]))
    for t in range(L):
        h = np.exp(Delta[:, t, :, None] * A[None]) * h + (Delta[:, t] * x[:, t])[:, :, None] * B[:, t, None, :]
    return Delta.sum(axis=1), h


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2 ** 31 - 1))
def test_combine_is_associative(seed):
    r = np.random.default_rng(seed)
    A = -np.exp(r.uniform(-2, 2, size=(3, 16)))
    cs = [(r.uniform(0, 3, size=(2, 3)), r.standard_normal((2, 3, 16))) for _ in range(3)]
    left = combine(A, combine(A, cs[0], cs[1]), cs[2])
    right = combine(A, cs[0], combine(A, cs[1], cs[2]))
    for a, b in zip(left, right):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_combine_matches_sequential_carry():
    r = np.random.default_rng(11)
    bt, L, D, N = 2, 40, 3, 16
    A = -np.exp(r.uniform(-1, 1, size=(D, N)))
    Delta = np.exp(r.uniform(-5, 0, size=(bt, L, D)))
    x = r.standard_normal((bt, L, D))
    B = r.standard_normal((bt, L, N))
    whole = chunk_carry(Delta, x, A, B)
    parts = combine(A, chunk_carry(Delta[:, :17], x[:, :17], A, B[:, :17]),
                    chunk_carry(Delta[:, 17:], x[:, 17:], A, B[:, 17:]))
    for a, b in zip(whole, parts):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def _chunked_scan(x, delta, A, B, C, Dskip, dt_bias, z, h0, Lc):
    """Three phases: local carries, exclusive combine seeded with h0, rescan from the true carry-in."""
    bt, L, D = x.shape
    N = A.shape[1]
    Delta = np.logaddexp(0.0, delta + dt_bias[None, None, :])
    bounds = [(s, min(L, s + Lc)) for s in range(0, L, Lc)]
    carries = [chunk_carry(Delta[:, a:b], x[:, a:b], A, B[:, a:b]) for a, b in bounds[:-1]]
    h_in = [np.zeros((bt, D, N)) if h0 is None else h0]
    acc = (np.zeros((bt, D)), h_in[0])
    for c in carries:
        acc = combine(A, acc, c)
        h_in.append(acc[1])
    ys, h = [], None
    for (a, b), hi in zip(bounds, h_in):
        y, h = oracle.recurrence(Delta[:, a:b], x[:, a:b], A, B[:, a:b], C[:, a:b], Dskip, hi)
        ys.append(y)
    y = np.concatenate(ys, axis=1)
    return y * oracle.silu(z), h


def test_chunked_scan_equals_oracle():
    r = np.random.default_rng(12)
    bt, L, D, N = 2, 203, 4, 16
    A = -np.exp(r.uniform(-1, 1.5, size=(D, N)))
    Dskip = r.uniform(0.5, 1.5, D)
    dt_bias = r.uniform(-5, -1, D)
    x, delta, z = (r.standard_normal((bt, L, D)) for _ in range(3))
    B, C = (r.standard_normal((bt, L, N)) for _ in range(2))
    h0 = r.standard_normal((bt, D, N))
    ref, href = oracle.scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=h0)
    for Lc in (1, 16, 64, 100, 202, 203, 500):
        y, h = _chunked_scan(x, delta, A, B, C, Dskip, dt_bias, z, h0, Lc)
        np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
        np.testing.assert_allclose(h, href, rtol=0, atol=1e-12 * np.abs(href).max())
