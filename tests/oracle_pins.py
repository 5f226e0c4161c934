"""Pins for the float64 oracle: results the pages and the mathematics fix.

Each pin takes an oracle module ``m`` (exposing softplus, silu, recurrence,
scan_fwd, state_update, scan_bwd, conv_silu and conv_scan_fwd) and raises AssertionError when ``m`` disagrees
with a value that does not come from ``m`` itself. The same pins run against
copies of the oracle with a planted mistake (tests/test_oracle_mutants.py),
which must each fail at least one of them.

Pages are cited by title and section.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.signal


def _rng(seed):
    return np.random.default_rng([391, seed])


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max|err| {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _sp(v):
    """softplus written independently of the oracle (log1p of exp, per element)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    it = np.nditer(v, flags=["multi_index"])
    for val in it:
        f = float(val)
        out[it.multi_index] = f + math.log1p(math.exp(-f)) if f > 0 else math.log1p(math.exp(f))
    return out


def _params(rng, D, N, A_mode="s4d"):
    if A_mode == "s4d":
        A = -(np.arange(N, dtype=np.float64) + 1.0)[None, :].repeat(D, 0)
    else:  # arbitrary negative diagonal, different per channel
        A = -np.exp(rng.uniform(-1.5, 1.5, size=(D, N)))
    Dskip = rng.uniform(0.5, 1.5, size=D)
    dt_bias = rng.uniform(-4.0, -1.0, size=D)
    return A, Dskip, dt_bias


# ---------------------------------------------------------------------------
# elementwise maps
# ---------------------------------------------------------------------------

def pin_softplus(m):
    """softplus(0) = ln 2; softplus(v) - softplus(-v) = v; log1p(exp) agreement."""
    assert abs(float(m.softplus(0.0)) - math.log(2.0)) < 1e-15
    v = np.linspace(-30, 30, 121)
    _close(m.softplus(v) - m.softplus(-v), v, 1e-14, "softplus odd part")
    _close(m.softplus(v), _sp(v), 1e-14, "softplus vs log1p(exp)")
    assert float(m.softplus(800.0)) == 800.0
    assert 0.0 < float(m.softplus(-700.0)) < 1e-300


def pin_silu(m):
    """silu(0) = 0; silu(z) - silu(-z) = z; silu = z * expit(z)."""
    import scipy.special
    assert float(m.silu(0.0)) == 0.0
    z = np.linspace(-40, 40, 161)
    _close(m.silu(z) - m.silu(-z), z, 1e-14, "silu odd part")
    _close(m.silu(z), z * scipy.special.expit(z), 1e-14, "silu vs z*expit(z)")
    assert abs(float(m.silu(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# ---------------------------------------------------------------------------
# (a) step size -> 0 passes the input through the skip term only
# ---------------------------------------------------------------------------

def pin_delta_zero_exact(m):
    """Delta = 0 exactly: Abar = 1 and Bbar = 0, so h stays h0 = 0 and y = D*x bit for bit.

    "DL0170 Mamba Selective SSM vs Attention", point (2): a small step leaves
    the state untouched and the token is ignored.
    """
    r = _rng(1)
    bt, L, D, N = 2, 37, 5, 16
    A, Dskip, _ = _params(r, D, N, "rand")
    x = r.standard_normal((bt, L, D))
    B = r.standard_normal((bt, L, N))
    C = r.standard_normal((bt, L, N))
    y, h = m.recurrence(np.zeros((bt, L, D)), x, A, B, C, Dskip, None)
    assert np.array_equal(y, Dskip[None, None, :] * x), "Delta=0 must give y = D*x exactly"
    assert np.array_equal(h, np.zeros((bt, D, N)))


def pin_delta_tiny_bias(m):
    """dt_bias = -60 gives Delta ~ 1e-26: y = D*x*silu(z) up to 1e-20 * max|x|."""
    r = _rng(2)
    bt, L, D, N = 2, 29, 3, 16
    A, Dskip, _ = _params(r, D, N)
    dt_bias = np.full(D, -60.0)
    x = r.standard_normal((bt, L, D))
    dl = 0.5 * r.standard_normal((bt, L, D))
    z = r.standard_normal((bt, L, D))
    B = r.standard_normal((bt, L, N))
    C = r.standard_normal((bt, L, N))
    out, h = m.scan_fwd(x, dl, A, B, C, Dskip, dt_bias, z=z)
    gate = z / (1.0 + np.exp(-z))
    expect = Dskip[None, None, :] * x * gate
    assert np.max(np.abs(out - expect)) <= 1e-20 * np.max(np.abs(x))
    assert np.max(np.abs(h)) <= 1e-20 * np.max(np.abs(x))
    assert np.max(np.abs(h)) > 0.0, "the state still receives the (tiny) input"


# ---------------------------------------------------------------------------
# (b) constant Delta, B, C: the layer is LTI and equals a convolution
# ---------------------------------------------------------------------------

def _lti_setup(seed, bt=2, L=160, D=3, N=16, A_mode="rand"):
    r = _rng(seed)
    A, Dskip, dt_bias = _params(r, D, N, A_mode)
    c_d = 0.5 * r.standard_normal(D)                 # constant delta per channel
    bvec = r.standard_normal((bt, N))
    cvec = r.standard_normal((bt, N))
    delta = np.broadcast_to(c_d[None, None, :], (bt, L, D)).copy()
    B = np.broadcast_to(bvec[:, None, :], (bt, L, N)).copy()
    C = np.broadcast_to(cvec[:, None, :], (bt, L, N)).copy()
    Delta = _sp(c_d + dt_bias)                       # (D,)
    Abar = np.exp(Delta[:, None] * A)                # (D, N)
    # convolution kernel K_d[k] = sum_n c_n * Abar_dn^k * Delta_d * b_n
    k = np.arange(L)
    K = np.einsum("bn,dnk,d,bn->bdk", cvec, Abar[:, :, None] ** k[None, None, :], Delta, bvec)
    return dict(A=A, Dskip=Dskip, dt_bias=dt_bias, delta=delta, B=B, C=C, Delta=Delta,
                Abar=Abar, K=K, bvec=bvec, cvec=cvec, bt=bt, L=L, D=D, N=N, r=r)


def pin_lti_direct(m):
    """LTI case equals the direct causal sum y_t = sum_k K[k] x_{t-k} + D x_t.

    "Mamba & State-Space Sequence Models", "Core mechanics" and "Self-check":
    with fixed Abar, Bbar, C the recurrence unrolls into one convolution.
    """
    s = _lti_setup(3)
    x = s["r"].standard_normal((s["bt"], s["L"], s["D"]))
    y, _ = m.scan_fwd(x, s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"])
    ref = np.empty_like(y)
    for b in range(s["bt"]):
        for d in range(s["D"]):
            for t in range(s["L"]):
                acc = 0.0
                for kk in range(t + 1):
                    acc += s["K"][b, d, kk] * x[b, t - kk, d]
                ref[b, t, d] = acc + s["Dskip"][d] * x[b, t, d]
    _close(y, ref, 1e-10, "LTI direct sum")


def pin_lti_fft(m):
    """LTI case equals the FFT convolution (zero padded to 2L), the textbook S4 route."""
    s = _lti_setup(4, L=257)
    x = s["r"].standard_normal((s["bt"], s["L"], s["D"]))
    y, _ = m.scan_fwd(x, s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"])
    L = s["L"]
    nfft = 2 * L
    Kf = np.fft.rfft(s["K"], nfft, axis=-1)                          # (bt, D, f)
    Xf = np.fft.rfft(np.transpose(x, (0, 2, 1)), nfft, axis=-1)     # (bt, D, f)
    conv = np.fft.irfft(Kf * Xf, nfft, axis=-1)[..., :L]
    ref = np.transpose(conv, (0, 2, 1)) + s["Dskip"][None, None, :] * x
    _close(y, ref, 1e-10, "LTI via FFT")


def pin_lti_closed_form(m):
    """x = 1: y_t = sum_n c_n Delta b_n (1 - Abar^(t+1)) / (1 - Abar) + D (geometric series)."""
    s = _lti_setup(5, L=300, A_mode="s4d")
    x = np.ones((s["bt"], s["L"], s["D"]))
    y, h = m.scan_fwd(x, s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"])
    t = np.arange(s["L"])
    Ab = s["Abar"]                                                   # (D, N)
    geo = (1.0 - Ab[None, :, :] ** (t[:, None, None] + 1)) / (1.0 - Ab[None, :, :])   # (L, D, N)
    ref = np.einsum("bn,tdn,d,bn->btd", s["cvec"], geo, s["Delta"], s["bvec"]) + s["Dskip"][None, None, :]
    _close(y, ref, 1e-10, "LTI closed form for x = 1")
    hL = np.einsum("dn,d,bn->bdn", geo[-1], s["Delta"], s["bvec"])
    _close(h, hL, 1e-10, "LTI closed-form final state")


def pin_lti_lfilter(m):
    """N = 1, constant Delta: h is the first-order IIR filter that scipy.signal.lfilter computes."""
    r = _rng(6)
    L = 400
    a = -np.array([[0.7]])
    Dskip = np.array([0.3])
    dt_bias = np.array([-1.2])
    c0 = 0.4
    delta = np.full((1, L, 1), c0)
    bval, cval = 1.7, -0.9
    B = np.full((1, L, 1), bval)
    C = np.full((1, L, 1), cval)
    x = r.standard_normal((1, L, 1))
    h0 = np.array([[[0.6]]])
    y, h = m.scan_fwd(x, delta, a, B, C, Dskip, dt_bias, h0=h0)
    Delta = _sp(np.array([c0 - 1.2]))[0]
    ab = math.exp(Delta * a[0, 0])
    zi = scipy.signal.lfiltic([Delta * bval], [1.0, -ab], y=[h0[0, 0, 0]])
    hs, _ = scipy.signal.lfilter([Delta * bval], [1.0, -ab], x[0, :, 0], zi=zi)
    ref = cval * hs + Dskip[0] * x[0, :, 0]
    _close(y[0, :, 0], ref, 1e-11, "lfilter")
    _close(h[0, 0, 0], hs[-1], 1e-11, "lfilter final state")


# ---------------------------------------------------------------------------
# (c) brute force: the causal matrix-mixer form
# ---------------------------------------------------------------------------

def brute_force(Delta, x, A, B, C, Dskip, h0=None):
    """y_t = sum_{s<=t} C_t (prod_{s<r<=t} Abar_r) Delta_s B_s x_s + D x_t (+ decayed h0).

    "Mamba", "Relation to Mamba-2" writes the layer as this causal matrix mixer
    (its symbols read as the discretised Abar and Bbar = Delta B). Explicit
    products, no recurrence.
    """
    bt, L, D = x.shape
    N = A.shape[1]
    Abar = np.exp(Delta[..., None] * A[None, None, :, :])            # (bt, L, D, N)
    y = np.zeros((bt, L, D))
    hL = np.zeros((bt, D, N))
    for t in range(L):
        for s in range(t + 1):
            P = np.ones((bt, D, N))
            for rr in range(s + 1, t + 1):
                P = P * Abar[:, rr]
            contrib = P * (Delta[:, s] * x[:, s])[:, :, None] * B[:, s, None, :]
            y[:, t] += np.einsum("bn,bdn->bd", C[:, t], contrib)
            if t == L - 1:
                hL += contrib
        if h0 is not None:
            P = np.ones((bt, D, N))
            for rr in range(0, t + 1):
                P = P * Abar[:, rr]
            y[:, t] += np.einsum("bn,bdn->bd", C[:, t], P * h0)
            if t == L - 1:
                hL += P * h0
        y[:, t] += Dskip[None, :] * x[:, t]
    return y, hL


def pin_brute_force(m):
    """The recurrence equals the causal matrix-mixer sum on tiny random inputs."""
    r = _rng(7)
    for (bt, L, D, N, with_h0) in [(2, 24, 3, 16, False), (1, 31, 4, 16, True), (2, 9, 2, 5, True)]:
        A, Dskip, dt_bias = _params(r, D, N, "rand")
        x = r.standard_normal((bt, L, D))
        dl = r.standard_normal((bt, L, D))
        B = r.standard_normal((bt, L, N))
        C = r.standard_normal((bt, L, N))
        h0 = r.standard_normal((bt, D, N)) if with_h0 else None
        Delta = _sp(dl + dt_bias[None, None, :])
        ref_y, ref_h = brute_force(Delta, x, A, B, C, Dskip, h0)
        y, h = m.scan_fwd(x, dl, A, B, C, Dskip, dt_bias, h0=h0)
        _close(y, ref_y, 1e-12, "brute force y")
        _close(h, ref_h, 1e-12, "brute force h_L")


# ---------------------------------------------------------------------------
# (d) overwrite limit, (e) pure decay
# ---------------------------------------------------------------------------

def pin_overwrite(m):
    """dt_bias = +200: Abar <= e^-200, so h_t = Delta_t B_t x_t and y_t = Delta_t (C_t.B_t) x_t + D x_t.

    "DL0170 Mamba Selective SSM vs Attention", point (2) and Figure 1: a large
    step forgets the old state and writes the new token.
    """
    r = _rng(8)
    bt, L, D, N = 2, 40, 3, 16
    A, Dskip, _ = _params(r, D, N)
    dt_bias = np.full(D, 200.0)
    x = r.standard_normal((bt, L, D))
    dl = r.standard_normal((bt, L, D))
    B = r.standard_normal((bt, L, N))
    C = r.standard_normal((bt, L, N))
    h0 = r.standard_normal((bt, D, N))
    y, h = m.scan_fwd(x, dl, A, B, C, Dskip, dt_bias, h0=h0)
    Delta = dl + 200.0
    cb = np.einsum("btn,btn->bt", C, B)
    ref = Delta * cb[:, :, None] * x + Dskip[None, None, :] * x
    _close(y, ref, 1e-12, "overwrite y")
    _close(h, (Delta[:, -1] * x[:, -1])[:, :, None] * B[:, -1, None, :], 1e-12, "overwrite h_L")


def pin_pure_decay(m):
    """x = 0, h0 != 0: h_t = exp(A * sum_{r<=t} Delta_r) h0 and y_t = C_t . h_t."""
    r = _rng(9)
    bt, L, D, N = 2, 50, 3, 16
    A, Dskip, dt_bias = _params(r, D, N, "rand")
    dl = r.standard_normal((bt, L, D))
    C = r.standard_normal((bt, L, N))
    B = r.standard_normal((bt, L, N))
    h0 = r.standard_normal((bt, D, N))
    y, h = m.scan_fwd(np.zeros((bt, L, D)), dl, A, B, C, Dskip, dt_bias, h0=h0)
    cum = np.cumsum(_sp(dl + dt_bias[None, None, :]), axis=1)          # (bt, L, D)
    hs = np.exp(cum[..., None] * A[None, None]) * h0[:, None]           # (bt, L, D, N)
    _close(y, np.einsum("btn,btdn->btd", C, hs), 1e-12, "pure decay y")
    _close(h, hs[:, -1], 1e-12, "pure decay h_L")


# ---------------------------------------------------------------------------
# (f) splitting and chained decode steps, (g) linearity, single token
# ---------------------------------------------------------------------------

def _random_case(seed, bt=2, L=45, D=4, N=16, gated=True):
    r = _rng(seed)
    A, Dskip, dt_bias = _params(r, D, N, "rand")
    return dict(x=r.standard_normal((bt, L, D)), delta=r.standard_normal((bt, L, D)),
                z=r.standard_normal((bt, L, D)) if gated else None,
                B=r.standard_normal((bt, L, N)), C=r.standard_normal((bt, L, N)),
                A=A, Dskip=Dskip, dt_bias=dt_bias, h0=r.standard_normal((bt, D, N)))


def pin_single_token(m):
    """One token from a zero state: out = (Delta (C.B) x + D x) silu(z), h = Delta B x."""
    s = _random_case(10, L=1)
    out, h = m.scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"], z=s["z"])
    Delta = _sp(s["delta"] + s["dt_bias"][None, None, :])
    cb = np.einsum("btn,btn->bt", s["C"], s["B"])[:, :, None]
    gate = s["z"] / (1.0 + np.exp(-s["z"]))
    _close(out, (Delta * cb * s["x"] + s["Dskip"] * s["x"]) * gate, 1e-14, "single token")
    _close(h, (Delta[:, 0] * s["x"][:, 0])[:, :, None] * s["B"][:, 0, None, :], 1e-14, "single token h")


def pin_split(m):
    """scan(0:L) = scan(L1:L, h0 = h_L1) after scan(0:L1), for several L1.

    h_0 is the initial condition the recurrence starts from ("DL0170 ...",
    "Mathematical Formulation"), so a sequence can be resumed from its state.
    """
    s = _random_case(11)
    args = lambda sl: (s["x"][:, sl], s["delta"][:, sl], s["A"], s["B"][:, sl], s["C"][:, sl],
                       s["Dskip"], s["dt_bias"])
    full, hfull = m.scan_fwd(*args(slice(None)), z=s["z"], h0=s["h0"])
    for L1 in (1, 7, 22, 44):
        a, ha = m.scan_fwd(*args(slice(0, L1)), z=s["z"][:, :L1], h0=s["h0"])
        b, hb = m.scan_fwd(*args(slice(L1, None)), z=s["z"][:, L1:], h0=ha)
        _close(np.concatenate([a, b], axis=1), full, 1e-13, f"split at {L1}")
        _close(hb, hfull, 1e-13, f"split state at {L1}")


def pin_chained_steps(m):
    """L chained single-token decode steps equal one scan ("Mamba & State-Space Sequence
    Models", "Core mechanics": inference runs the recurrence one step at a time)."""
    s = _random_case(12, L=20)
    full, hfull = m.scan_fwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"],
                             z=s["z"], h0=s["h0"])
    h = s["h0"].copy()
    h_before = h.copy()
    for t in range(s["x"].shape[1]):
        out, h = m.state_update(h, s["x"][:, t], s["delta"][:, t], s["A"], s["B"][:, t], s["C"][:, t],
                                s["Dskip"], s["dt_bias"], z=s["z"][:, t])
        _close(out, full[:, t], 1e-13, f"decode step {t}")
    assert np.array_equal(s["h0"], h_before), "state_update must not modify its input state"
    _close(h, hfull, 1e-13, "decode chain final state")


def pin_linearity(m):
    """Ungated, fixed delta, B, C: (y, h_L) is linear in (x, h0)."""
    s1 = _random_case(13, gated=False)
    s2 = _random_case(14, gated=False)
    al, be = 0.7, -1.3
    f = lambda x, h0: m.scan_fwd(x, s1["delta"], s1["A"], s1["B"], s1["C"], s1["Dskip"],
                                 s1["dt_bias"], h0=h0)
    y1, h1 = f(s1["x"], s1["h0"])
    y2, h2 = f(s2["x"], s2["h0"])
    y3, h3 = f(al * s1["x"] + be * s2["x"], al * s1["h0"] + be * s2["h0"])
    _close(y3, al * y1 + be * y2, 1e-12, "linearity y")
    _close(h3, al * h1 + be * h2, 1e-12, "linearity h")


# ---------------------------------------------------------------------------
# (h) the backward pass
# ---------------------------------------------------------------------------

_GRAD_INPUTS = ("x", "delta", "z", "A", "B", "C", "Dskip", "dt_bias", "h0")


def _bf_objective(p, dout, dh_last):
    """J = sum(dout * out) + sum(dh_last * h_L), through the brute-force sum.

    Written independently of the oracle: its own softplus, its own gate and
    the explicit causal-matrix form above.
    """
    Delta = _sp(p["delta"] + p["dt_bias"][None, None, :])
    y, hL = brute_force(Delta, p["x"], p["A"], p["B"], p["C"], p["Dskip"], p["h0"])
    if p.get("z") is not None:
        y = y * (p["z"] / (1.0 + np.exp(-p["z"])))
    J = float(np.sum(dout * y))
    if dh_last is not None:
        J += float(np.sum(dh_last * hL))
    return J


def _bwd_case(seed, bt, L, D, N, gated=True, with_h0=True, with_dh=True):
    r = _rng(seed)
    A, Dskip, dt_bias = _params(r, D, N, "rand")
    p = dict(x=r.standard_normal((bt, L, D)), delta=r.standard_normal((bt, L, D)),
             z=r.standard_normal((bt, L, D)) if gated else None,
             B=r.standard_normal((bt, L, N)), C=r.standard_normal((bt, L, N)),
             A=A, Dskip=Dskip, dt_bias=dt_bias + 1.5,   # steps near 0.1-1: decay and input both matter
             h0=r.standard_normal((bt, D, N)) if with_h0 else None)
    dout = r.standard_normal((bt, L, D))
    dh = r.standard_normal((bt, D, N)) if with_dh else None
    return p, dout, dh


def _oracle_bwd(m, p, dout, dh):
    return m.scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["Dskip"], p["dt_bias"], dout,
                      z=p["z"], h0=p["h0"], dh_last=dh)


def pin_bwd_finite_differences(m):
    """Every gradient equals central finite differences of the brute-force objective.

    Steps of 1e-6 in float64 leave a truncation error near 1e-12 and a rounding
    error near 1e-10 of the objective's size, far inside the 1e-6 bound.
    """
    for seed, shape, gated, with_h0, with_dh in [(20, (2, 6, 2, 3), True, True, True),
                                                 (21, (1, 5, 3, 4), False, False, False)]:
        p, dout, dh = _bwd_case(seed, *shape, gated=gated, with_h0=with_h0, with_dh=with_dh)
        g = _oracle_bwd(m, p, dout, dh)
        if not gated:
            assert g["z"] is None, "ungated scan has no gate gradient"
        for name in _GRAD_INPUTS:
            if p.get(name) is None:
                if name == "h0":       # gradient at h0 = 0
                    base = dict(p, h0=np.zeros((shape[0], shape[2], shape[3])))
                else:
                    continue
            else:
                base = p
            fd = np.zeros_like(base[name])
            for idx in np.ndindex(*base[name].shape):
                eps = 1e-6 * max(1.0, abs(base[name][idx]))
                hi = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
                lo = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
                hi[name][idx] += eps
                lo[name][idx] -= eps
                fd[idx] = (_bf_objective(hi, dout, dh) - _bf_objective(lo, dout, dh)) / (2 * eps)
            _close(g[name], fd, 1e-6, f"finite differences d{name} (case {seed})")


def pin_bwd_dot_products(m):
    """Exact identities where J is affine in an input: J(X) - J(X = 0) = <dJ/dX, X>.

    With the other inputs fixed, out and h_L are linear in x (with h0 = 0), in
    B, in C, in Dskip and in h0 (with x = 0), so the identity holds up to
    rounding, at a length no finite difference would reach as precisely.
    """
    p, dout, dh = _bwd_case(22, 2, 24, 3, 16)
    zero = lambda **kw: dict(p, **kw)
    xz = np.zeros_like(p["x"])
    cases = [("x", zero(h0=None), zero(h0=None, x=xz)),
             ("B", p, zero(B=np.zeros_like(p["B"]))),
             ("C", p, zero(C=np.zeros_like(p["C"]))),
             ("Dskip", p, zero(Dskip=np.zeros_like(p["Dskip"]))),
             ("h0", zero(x=xz), zero(x=xz, h0=np.zeros_like(p["h0"])))]
    for name, at, at0 in cases:
        g = _oracle_bwd(m, at, dout, dh)
        lhs = _bf_objective(at, dout, dh) - _bf_objective(at0, dout, dh)
        rhs = float(np.sum(g[name] * at[name]))
        assert abs(lhs - rhs) <= 1e-11 * max(abs(lhs), 1.0), f"dot product d{name}: {lhs!r} vs {rhs!r}"


def pin_bwd_lti_transpose(m):
    """Constant step, B and C, ungated: y = K * x + D x is a causal convolution, so
    dJ/dx is the correlation of dout with K plus D dout, and dJ/dh0_n is
    sum_t dout_t C_n exp((t + 1) Delta A_n) (the S4 convolution view the pages
    contrast Mamba with: "DL0170 ...", point (3))."""
    r = _rng(23)
    bt, L, D, N = 1, 64, 2, 16
    A, Dskip, dt_bias = _params(r, D, N, "rand")
    Bv = r.standard_normal(N)
    Cv = r.standard_normal(N)
    x = r.standard_normal((bt, L, D))
    h0 = r.standard_normal((bt, D, N))
    dout = r.standard_normal((bt, L, D))
    g = m.scan_bwd(x, np.zeros((bt, L, D)), A, np.tile(Bv, (bt, L, 1)), np.tile(Cv, (bt, L, 1)),
                   Dskip, dt_bias, dout, h0=h0)
    Delta = _sp(dt_bias)
    k = np.arange(L, dtype=np.float64)
    for d in range(D):
        decay = np.exp(np.outer(k, Delta[d] * A[d]))                     # (L, N): exp(k Delta A)
        K = decay @ (Cv * Delta[d] * Bv)
        go = dout[0, :, d]
        ref = np.convolve(go[::-1], K)[:L][::-1] + Dskip[d] * go
        _close(g["x"][0, :, d], ref, 1e-12, f"LTI transposed convolution, channel {d}")
        ref_h0 = (decay * np.exp(Delta[d] * A[d])[None, :]).T @ go * Cv
        _close(g["h0"][0, d], ref_h0, 1e-12, f"LTI dh0, channel {d}")


def pin_bwd_split(m):
    """Backward of scan(0:L) = backward of scan(L1:L) then of scan(0:L1), the
    second receiving the first's starting-state gradient as its dh_last."""
    p, dout, dh = _bwd_case(24, 2, 30, 3, 16)
    whole = _oracle_bwd(m, p, dout, dh)
    for L1 in (1, 13, 29):
        a = {k: (v[:, :L1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in p.items()}
        b = {k: (v[:, L1:] if k in ("x", "delta", "z", "B", "C") else v) for k, v in p.items()}
        _, hmid = m.scan_fwd(a["x"], a["delta"], p["A"], a["B"], a["C"], p["Dskip"], p["dt_bias"], h0=p["h0"])
        b["h0"] = hmid
        gb = _oracle_bwd(m, b, dout[:, L1:], dh)
        ga = _oracle_bwd(m, a, dout[:, :L1], gb["h0"])
        for k in ("x", "delta", "z", "B", "C"):
            _close(np.concatenate([ga[k], gb[k]], axis=1), whole[k], 1e-12, f"split {L1} d{k}")
        for k in ("A", "Dskip", "dt_bias"):
            _close(ga[k] + gb[k], whole[k], 1e-12, f"split {L1} d{k}")
        _close(ga["h0"], whole["h0"], 1e-12, f"split {L1} dh0")


# ---------------------------------------------------------------------------
# (i) the local convolution before the scan
# ---------------------------------------------------------------------------

def _silu_ref(v):
    return v / (1.0 + np.exp(-v))


def _conv_case(seed, bt=2, L=37, D=3, K=4, with_init=True):
    r = _rng(seed)
    return dict(xin=r.standard_normal((bt, L, D)), w=r.standard_normal((D, K)), b=r.standard_normal(D),
                init=r.standard_normal((bt, K - 1, D)) if (with_init and K > 1) else None)


def pin_conv_numpy_convolve(m):
    """Pre-activation = bias + numpy.convolve of [init, xin] with the reversed taps ('valid' part)."""
    for K in (1, 2, 3, 4):
        c = _conv_case(30 + K, K=K, with_init=K > 1)
        out = m.conv_silu(c["xin"], c["w"], c["b"], c["init"])
        bt, L, D = c["xin"].shape
        for bi in range(bt):
            for d in range(D):
                head = c["init"][bi, :, d] if c["init"] is not None else np.zeros(K - 1)
                seq = np.concatenate([head, c["xin"][bi, :, d]])
                v = c["b"][d] + np.convolve(seq, c["w"][d, ::-1], mode="valid")
                _close(out[bi, :, d], _silu_ref(v), 1e-13, f"conv K={K} b={bi} d={d}")


def pin_conv_lfilter(m):
    """The same as an FIR filter (scipy.signal.lfilter) over [init, xin], first K-1 outputs dropped."""
    c = _conv_case(35, K=4)
    out = m.conv_silu(c["xin"], c["w"], c["b"], c["init"])
    for bi in range(2):
        for d in range(3):
            seq = np.concatenate([c["init"][bi, :, d], c["xin"][bi, :, d]])
            v = scipy.signal.lfilter(c["w"][d, ::-1], [1.0], seq)[3:] + c["b"][d]
            _close(out[bi, :, d], _silu_ref(v), 1e-13, f"lfilter b={bi} d={d}")


def pin_conv_impulse_and_causality(m):
    """A unit impulse at t0 gives silu(w_{K-1-j}) at t0 + j, silu(0) = 0 elsewhere; later inputs
    never change earlier outputs."""
    K, L = 4, 20
    w = _rng(36).standard_normal((1, K))
    for t0 in (0, 5, L - 2):
        xin = np.zeros((1, L, 1))
        xin[0, t0, 0] = 1.0
        out = m.conv_silu(xin, w, np.zeros(1))[0, :, 0]
        ref = np.zeros(L)
        for j in range(K):
            if t0 + j < L:
                ref[t0 + j] = _silu_ref(w[0, K - 1 - j])
        _close(out, ref, 1e-15, f"impulse at {t0}")
    c = _conv_case(37)
    base = m.conv_silu(c["xin"], c["w"], c["b"], c["init"])
    x2 = c["xin"].copy()
    x2[:, 20:] += 5.0
    moved = m.conv_silu(x2, c["w"], c["b"], c["init"])
    assert np.array_equal(base[:, :20], moved[:, :20]), "an output depends on a later input"
    assert not np.allclose(base[:, 20:23], moved[:, 20:23]), "the perturbed inputs must matter"


def pin_conv_scan_split_and_identity(m):
    """conv_scan over [0, L) = conv_scan over [L1, L) resumed from (h_L1, the last K-1 inputs);
    identity taps (0, 0, 0, 1) with zero bias give scan_fwd(silu(xin))."""
    c = _conv_case(38, L=40, D=3)
    s = _random_case(39, L=40, D=3)
    run = lambda sl, init, h0: m.conv_scan_fwd(c["xin"][:, sl], c["w"], c["b"], s["delta"][:, sl], s["A"],
                                               s["B"][:, sl], s["C"][:, sl], s["Dskip"], s["dt_bias"],
                                               z=s["z"][:, sl], h0=h0, conv_init=init)
    full, hf = run(slice(None), c["init"], s["h0"])
    for L1 in (3, 17, 39):
        a, ha = run(slice(0, L1), c["init"], s["h0"])
        tail = np.concatenate([c["init"], c["xin"][:, :L1]], axis=1)[:, -3:]
        b, hb = run(slice(L1, None), tail, ha)
        _close(np.concatenate([a, b], axis=1), full, 1e-13, f"conv scan split at {L1}")
        _close(hb, hf, 1e-13, f"conv scan split state at {L1}")
    w_id = np.zeros((3, 4))
    w_id[:, 3] = 1.0
    y1, h1 = m.conv_scan_fwd(c["xin"], w_id, np.zeros(3), s["delta"], s["A"], s["B"], s["C"], s["Dskip"],
                             s["dt_bias"], z=s["z"], h0=s["h0"], conv_init=c["init"])
    y2, h2 = m.scan_fwd(_silu_ref(c["xin"]), s["delta"], s["A"], s["B"], s["C"], s["Dskip"], s["dt_bias"],
                        z=s["z"], h0=s["h0"])
    _close(y1, y2, 1e-14, "identity taps")
    _close(h1, h2, 1e-14, "identity taps state")


def pin_conv_chained_steps(m):
    """Chained convolution decode steps (conv state of the last K-1 inputs) equal one conv scan."""
    c = _conv_case(40, L=15, D=3)
    s = _random_case(41, L=15, D=3)
    full, hf = m.conv_scan_fwd(c["xin"], c["w"], c["b"], s["delta"], s["A"], s["B"], s["C"], s["Dskip"],
                               s["dt_bias"], z=s["z"], h0=s["h0"], conv_init=c["init"])
    cs, h = c["init"].copy(), s["h0"].copy()
    for t in range(15):
        before = cs.copy()
        out, h, cs = m.conv_state_update(cs, h, c["xin"][:, t], c["w"], c["b"], s["delta"][:, t], s["A"],
                                         s["B"][:, t], s["C"][:, t], s["Dskip"], s["dt_bias"], z=s["z"][:, t])
        _close(out, full[:, t], 1e-13, f"conv decode step {t}")
        assert np.array_equal(cs[:, :-1], before[:, 1:]) and np.array_equal(cs[:, -1], c["xin"][:, t]), \
            "the conv state must shift by one input"
    _close(h, hf, 1e-13, "conv decode chain final state")


PINS = [pin_softplus, pin_silu, pin_delta_zero_exact, pin_delta_tiny_bias, pin_lti_direct,
        pin_lti_fft, pin_lti_closed_form, pin_lti_lfilter, pin_brute_force, pin_overwrite,
        pin_pure_decay, pin_single_token, pin_split, pin_chained_steps, pin_linearity,
        pin_bwd_finite_differences, pin_bwd_dot_products, pin_bwd_lti_transpose, pin_bwd_split,
        pin_conv_numpy_convolve, pin_conv_lfilter, pin_conv_impulse_and_causality, pin_conv_scan_split_and_identity,
        pin_conv_chained_steps]
