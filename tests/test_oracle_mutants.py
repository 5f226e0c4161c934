"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Every mutant is the oracle's own source with one plausible slip (a dropped
term, a wrong sign, a wrong index, a swapped operand, a wrong function).
The copy is built on the CPU in a fresh module; the real oracle is untouched.
"""
import inspect
import types

import pytest

import oracle.s6 as s6
from oracle_pins import PINS

SRC = inspect.getsource(s6)

MUTANTS = {
    "readout-before-update": (
        "        h = Abar * h + Bbar_x\n"
        "        y[:, t, :] = np.einsum(\"bdn,bn->bd\", h, C[:, t, :]) + Dskip[None, :] * x[:, t, :]\n",
        "        y[:, t, :] = np.einsum(\"bdn,bn->bd\", h, C[:, t, :]) + Dskip[None, :] * x[:, t, :]\n"
        "        h = Abar * h + Bbar_x\n"),
    "input-term-without-delta": ("(Delta[:, t, :] * x[:, t, :])[:, :, None]", "(x[:, t, :])[:, :, None]"),
    "decay-sign-flipped": ("np.exp(Delta[:, t, :, None] * A[None, :, :])",
                           "np.exp(-Delta[:, t, :, None] * A[None, :, :])"),
    "decay-without-delta": ("np.exp(Delta[:, t, :, None] * A[None, :, :])",
                            "np.exp(A[None, :, :] + 0 * Delta[:, t, :, None])"),
    "states-of-A-reversed": ("A[None, :, :])", "A[None, :, ::-1])"),
    "B-and-C-swapped": ("* B[:, t, None, :]", "* C[:, t, None, :]"),
    "readout-uses-B": ("h, C[:, t, :])", "h, B[:, t, :])"),
    "readout-previous-C": ("h, C[:, t, :])", "h, C[:, max(t - 1, 0), :])"),
    "skip-dropped": (" + Dskip[None, :] * x[:, t, :]", ""),
    "skip-on-previous-token": ("Dskip[None, :] * x[:, t, :]", "Dskip[None, :] * x[:, max(t - 1, 0), :]"),
    "softplus-is-relu": ("return np.logaddexp(0.0, v)", "return np.maximum(v, 0.0)"),
    "softplus-is-exp": ("return np.logaddexp(0.0, v)", "return np.exp(v)"),
    "dt-bias-dropped": ("np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, None, :]",
                        "np.asarray(delta, dtype=np.float64)"),
    "dt-bias-subtracted": ("np.asarray(delta, dtype=np.float64) + np.asarray(dt_bias",
                           "np.asarray(delta, dtype=np.float64) - np.asarray(dt_bias"),
    "gate-is-sigmoid": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "gate-sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "h0-ignored": ("h = np.zeros((bt, D, N)) if h0 is None else np.array(h0, dtype=np.float64)",
                   "h = np.zeros((bt, D, N))"),
    "state-update-ignores-state": ("y, hn = scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=zz, h0=h)",
                                   "y, hn = scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=zz, h0=None)"),
    "state-update-ungated": ("y, hn = scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=zz, h0=h)",
                             "y, hn = scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=None, h0=h)"),
    "gate-before-skip": ("    if z is not None:\n        y = y * silu(z)\n",
                         "    if z is not None:\n        y = (y - Dskip * x) * silu(z) + Dskip * x\n"),
    # the backward pass
    "bwd-carry-not-decayed": ("        carry = Abar * mu\n", "        carry = mu\n"),
    "bwd-decay-term-uses-new-state": ("w = mu * Abar * hs[:, t]", "w = mu * Abar * hs[:, t + 1]"),
    "bwd-dx-skip-dropped": ("dx[:, t] = du * Delta[:, t] + dy[:, t] * Dskip[None, :]", "dx[:, t] = du * Delta[:, t]"),
    "bwd-dx-skip-uses-dout": ("dx[:, t] = du * Delta[:, t] + dy[:, t] * Dskip[None, :]",
                              "dx[:, t] = du * Delta[:, t] + dout[:, t] * Dskip[None, :]"),
    "bwd-ddelta-input-term-dropped": ("dDelta[:, t] = du * x[:, t] + ", "dDelta[:, t] = "),
    "bwd-ddelta-decay-term-dropped": ("dDelta[:, t] = du * x[:, t] + np.einsum(\"bdn,dn->bd\", w, A)",
                                      "dDelta[:, t] = du * x[:, t]"),
    "bwd-softplus-derivative-dropped": ("dv = dDelta * _sigmoid(v)", "dv = dDelta"),
    "bwd-dz-silu-derivative-truncated": ("dz = dout * y * sg * (1.0 + z * (1.0 - sg))", "dz = dout * y * sg"),
    "bwd-dy-ignores-gate": ("dy = dout * z * sg", "dy = dout"),
    "bwd-dC-previous-state": ("dC = np.einsum(\"btd,btdn->btn\", dy, hs[:, 1:])",
                              "dC = np.einsum(\"btd,btdn->btn\", dy, hs[:, :-1])"),
    "bwd-dB-without-delta": ("np.einsum(\"bdn,bd->bn\", mu, Delta[:, t] * x[:, t])",
                             "np.einsum(\"bdn,bd->bn\", mu, x[:, t])"),
    "bwd-dA-without-delta": ("dA += np.einsum(\"bdn,bd->dn\", w, Delta[:, t])",
                             "dA += np.einsum(\"bdn,bd->dn\", w, np.ones_like(Delta[:, t]))"),
    "bwd-dh-last-ignored": ("carry = np.zeros((bt, D, N)) if dh_last is None else np.array(dh_last, dtype=np.float64)",
                            "carry = np.zeros((bt, D, N))"),
    "bwd-dh0-undecayed": ("dt_bias=dv.sum(axis=(0, 1)), h0=carry)", "dt_bias=dv.sum(axis=(0, 1)), h0=mu)"),
    "bwd-adjoint-reads-B": ("mu = dy[:, t, :, None] * C[:, t, None, :] + carry",
                            "mu = dy[:, t, :, None] * B[:, t, None, :] + carry"),
    "bwd-du-reads-C": ("du = np.einsum(\"bdn,bn->bd\", mu, B[:, t])", "du = np.einsum(\"bdn,bn->bd\", mu, C[:, t])"),
    "bwd-dDskip-uses-dout": ("Dskip=np.einsum(\"btd,btd->d\", dy, x)", "Dskip=np.einsum(\"btd,btd->d\", dout, x)"),
    "bwd-dbias-before-softplus-derivative": ("dt_bias=dv.sum(axis=(0, 1))", "dt_bias=dDelta.sum(axis=(0, 1))"),
    "bwd-dz-ungated-output": ("dz = dout * y * sg", "dz = dout * (y - Dskip * x) * sg"),
    # the local convolution
    "conv-taps-reversed": ("v[:, t, :] += w[None, :, k] * padded[:, t + k, :]",
                           "v[:, t, :] += w[None, :, K - 1 - k] * padded[:, t + k, :]"),
    "conv-window-shifted": ("v[:, t, :] += w[None, :, k] * padded[:, t + k, :]",
                            "v[:, t, :] += w[None, :, k] * padded[:, min(t + k + 1, L + K - 2), :]"),
    "conv-bias-dropped": ("v = np.broadcast_to(b, (bt, L, D)).copy()", "v = np.zeros((bt, L, D))"),
    "conv-no-activation": ("    return silu(v)\n\n\ndef conv_scan_fwd", "    return v\n\n\ndef conv_scan_fwd"),
    "conv-init-ignored": ("head = np.zeros((bt, K - 1, D)) if conv_init is None else np.asarray(conv_init, dtype=np.float64)",
                          "head = np.zeros((bt, K - 1, D))"),
    "conv-init-reversed": ("else np.asarray(conv_init, dtype=np.float64)",
                           "else np.asarray(conv_init, dtype=np.float64)[:, ::-1]"),
    "conv-scan-ignores-gate": ("    return scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=h0)",
                               "    return scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=None, h0=h0)"),
    "conv-decode-state-not-shifted": ("    return y[:, 0, :], hn, both[:, 1:]", "    return y[:, 0, :], hn, both[:, :-1]"),
    "conv-decode-ignores-state": ("h0=h, conv_init=conv_state, io=io)", "h0=h, conv_init=None, io=io)"),
    "conv-scan-ignores-h0": ("    return scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=h0)",
                             "    return scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=None)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = SRC.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _fails(pin, mod):
    try:
        pin(mod)
    except Exception:  # an assertion, or a crash the slip causes
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = [p.__name__ for p in PINS if _fails(p, mod)]
    assert caught, f"no pin catches the planted mistake {name!r}"
