"""The C ABI driven from plain C++ (hipMalloc'd buffers, no Python, no torch) on
the GPU: tests/c_abi/scan_demo runs a scan and a decode step and writes its
inputs and outputs; the float64 oracle recomputes every output from the same
bits (needs an MI355X and the demo, which build() compiles)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_util import TOL, assert_close, log
from selective_state_space_39_amd import build as b

pytestmark = pytest.mark.gpu


def test_c_abi_consumer(tmp_path):
    assert os.path.exists(b.DEMO), f"{b.DEMO} is missing: build() compiles it"
    log(f"running {b.DEMO}")
    r = subprocess.run([b.DEMO, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"scan_demo failed: {r.stdout}{r.stderr}"
    log(r.stdout.strip())
    batch, L, D, N = 2, 300, 40, 16
    ld = lambda name, *shape: np.fromfile(tmp_path / f"{name}.f32", dtype=np.float32).reshape(shape)
    x, delta, z = ld("x", batch, L, D), ld("delta", batch, L, D), ld("z", batch, L, D)
    B, C = ld("B", batch, L, N), ld("C", batch, L, N)
    A, Dskip, dt_bias, h0 = ld("A", D, N), ld("Dskip", D), ld("dt_bias", D), ld("h0", batch, D, N)
    ry, rh = oracle.scan_fwd(x, delta, A, B, C, Dskip, dt_bias, z=z, h0=h0, io="f32")
    assert_close(ld("y", batch, L, D), ry, TOL["f32"], "C ABI scan y")
    hL = ld("h_last", batch, D, N)
    assert_close(hL, rh, TOL["f32"], "C ABI scan h_L")
    # the decode step started from the library's own h_L
    ry1, rh1 = oracle.state_update(hL, ld("x1", batch, D), ld("delta1", batch, D), A, ld("B1", batch, N),
                                   ld("C1", batch, N), Dskip, dt_bias, z=ld("z1", batch, D), io="f32")
    assert_close(ld("y1", batch, D), ry1, TOL["f32"], "C ABI decode y")
    assert_close(ld("h1", batch, D, N), rh1, TOL["f32"], "C ABI decode h")
