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
