"""The float64 SSD oracle against its pins, planted mistakes, and the chunked
(intra-chunk masked product + carried state) evaluation the GPU kernel uses."""
import inspect
import types

import numpy as np
import pytest

import oracle.ssd as ssd
from oracle_pins import _close, _sp
from ssd_pins import SSD_PINS, ssd_case


@pytest.mark.parametrize("pin", SSD_PINS, ids=[p.__name__ for p in SSD_PINS])
def test_pin(pin):
    pin(ssd)


SRC = inspect.getsource(ssd)
MUTANTS = {
    "readout-before-update": ("        h = decay[:, :, None, None] * h + inp\n"
                              "        y[:, t] = np.einsum(\"bhpn,bn->bhp\", h, C[:, t]) + Dskip[None, :, None] * x[:, t]\n",
                              "        y[:, t] = np.einsum(\"bhpn,bn->bhp\", h, C[:, t]) + Dskip[None, :, None] * x[:, t]\n"
                              "        h = decay[:, :, None, None] * h + inp\n"),
    "input-without-delta": ("inp = (Delta[:, t, :, None] * x[:, t])", "inp = (x[:, t])"),
    "decay-sign": ("decay = np.exp(Delta[:, t] * A[None, :])", "decay = np.exp(-Delta[:, t] * A[None, :])"),
    "decay-shared-across-heads": ("decay = np.exp(Delta[:, t] * A[None, :])",
                                  "decay = np.exp(Delta[:, t, :1] * A[None, :])"),
    "B-and-C-swapped": ("* B[:, t, None, None, :]", "* C[:, t, None, None, :]"),
    "skip-dropped": (" + Dskip[None, :, None] * x[:, t]", ""),
    "bias-dropped": ("np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, None, :]",
                     "np.asarray(delta, dtype=np.float64)"),
    "gate-dropped": ("        y = y * silu(z)\n", "        y = y\n"),
    "h0-ignored": ("h = np.zeros((bt, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64)",
                   "h = np.zeros((bt, H, P, N))"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, name
    mod = types.ModuleType("ssd_mutant_" + name.replace("-", "_"))
    mod.__dict__["__package__"] = "oracle"
    exec(compile(SRC.replace(old, new, 1), f"<ssd mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in SSD_PINS:
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches {name!r}"


# ---------------------------------------------------------------------------
# the chunked evaluation, in float64 (independent of any GPU code)
# ---------------------------------------------------------------------------

def chunked_ssd(x, delta, A, B, C, Dskip, dt_bias, z, h0, Q):
    """Per chunk of Q tokens, with S_t = A * (sum of Delta up to t inside the chunk):
    y = ((C B^T) * Lmask) (Delta x) + exp(S_t) C state_in^T + D x, where
    Lmask[t, i] = exp(S_t - S_i) for i <= t; then
    state_out = exp(S_end) state_in + sum_i exp(S_end - S_i) Delta_i x_i B_i^T."""
    bt, L, H, P = x.shape
    N = B.shape[-1]
    Delta = _sp(delta + dt_bias[None, None, :])
    y = np.empty((bt, L, H, P))
    state = np.zeros((bt, H, P, N)) if h0 is None else h0.copy()
    for c0 in range(0, L, Q):
        c1 = min(L, c0 + Q)
        for b in range(bt):
            G = C[b, c0:c1] @ B[b, c0:c1].T                                     # (q, q), shared by heads
            for h in range(H):
                S = np.cumsum(Delta[b, c0:c1, h]) * A[h]                           # (q,)
                Lm = np.tril(np.exp(S[:, None] - S[None, :]))
                xd = Delta[b, c0:c1, h, None] * x[b, c0:c1, h]                     # (q, P)
                yd = (G * Lm) @ xd
                yo = np.exp(S)[:, None] * (C[b, c0:c1] @ state[b, h].T)
                y[b, c0:c1, h] = yd + yo + Dskip[h] * x[b, c0:c1, h]
                w = np.exp(S[-1] - S) * Delta[b, c0:c1, h]                         # (q,)
                state[b, h] = np.exp(S[-1]) * state[b, h] + (w[:, None] * x[b, c0:c1, h]).T @ B[b, c0:c1]
    if z is not None:
        y = y * (z / (1.0 + np.exp(-z)))
    return y, state


@pytest.mark.parametrize("Q", [1, 4, 7, 16, 64])
def test_chunked_evaluation_equals_oracle(Q):
    c = ssd_case(4, L=45, H=3, P=5, N=6)
    y, h = ssd.ssd_fwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["Dskip"], c["dt_bias"], z=c["z"], h0=c["h0"])
    yc, hc = chunked_ssd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["Dskip"], c["dt_bias"], c["z"], c["h0"], Q)
    _close(yc, y, 1e-12, f"chunked Q={Q} y")
    _close(hc, h, 1e-12, f"chunked Q={Q} h")
