"""HIP library vs the float64 oracle on the same seeded inputs (needs an MI355X).

Bounds: max|err| <= 1e-4 * max|ref| for float32 io, <= 2e-2 * max|ref| for
bfloat16 io, on the gated output y and on the final state h_L (the same
relative bound, normalised by max|h_ref|).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, dev, f32dev, gpu_scan, host64, log, oracle_scan
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _check_scan(s, chunk_len=0, gated=True, h0=None, channels=None, what=""):
    log(f"case {what}: shape {s.shape} io {s.io} chunk_len {chunk_len} gated {gated} h0 {h0 is not None} "
        f"plan {binding.plan(s.shape[0], s.shape[1], s.shape[2], 1 if s.io == 'bf16' else 0, chunk_len)}")
    y, h = gpu_scan(s, chunk_len=chunk_len, h0=h0, gated=gated)
    ref_y, ref_h = oracle_scan(s, channels=channels, h0=h0, gated=gated)
    yy, hh = host64(y), host64(h)
    if channels is not None:
        yy, hh = yy[:, :, channels], hh[:, channels]
    tol = TOL[s.io]
    ey = assert_close(yy, ref_y, tol, f"{what} y")
    eh = assert_close(hh, ref_h, tol, f"{what} h_L")
    return ey, eh


def test_tiny_f32():
    """1 x 256 x 16, every tensor float32."""
    s = inputs.make_workload("tiny-f32")
    _check_scan(s, what="tiny-f32")


@pytest.mark.parametrize("batch,L,D,chunk,gated,h0,io", [
    (1, 1, 16, 0, True, False, "bf16"),          # one token
    (2, 300, 200, 64, True, True, "bf16"),        # ragged L and D, several chunks and tiles
    (3, 37, 5, 32, False, False, "bf16"),         # tiny D, ungated
    (1, 1000, 130, 0, True, True, "bf16"),        # automatic plan
    (2, 513, 64, 96, True, True, "f32"),          # f32 io, ragged last chunk
    (1, 97, 257, 32, False, True, "f32"),
    (2, 2048, 256, 2048, True, False, "bf16"),    # one chunk, full-length ring
])
def test_small_cases(batch, L, D, chunk, gated, h0, io):
    s = inputs.make_scan_inputs(batch, L, D, io=io, seed=(39, 1000 + L + D), gated=gated, with_h0=h0)
    _check_scan(s, chunk_len=chunk, gated=gated, h0=s.h0, what=f"small {batch}x{L}x{D}")


def test_mamba130m_layer_full():
    """8 x 2048 x 1536, bf16, every output."""
    s = inputs.make_workload("mamba-130m-layer")
    _check_scan(s, what="mamba-130m-layer")


def test_mamba28b_layer_full():
    """4 x 2048 x 5120, bf16, every output."""
    s = inputs.make_workload("mamba-2.8b-layer")
    _check_scan(s, what="mamba-2.8b-layer")


def test_long_context_128k_sampled_channels():
    """Long context: every token of 64 sampled channels (spread over the chunk
    groups, first and last channel included) against the oracle."""
    s = inputs.make_workload("long-context-128k")
    r = np.random.default_rng(4)
    ch = np.unique(np.concatenate([[0, 1, 63, 64, 1023, 1024, 2046, 2047], r.choice(2048, 56, replace=False)]))
    _check_scan(s, channels=ch, what="long-context-128k")


def test_decode_256x5120_chain():
    """1000 chained decode steps: y and the state of a 16 x 256 sample of
    (batch row, channel) pairs against the oracle's own float64 chain, which
    starts from the same float32 state and is never re-seeded from the GPU."""
    batch, Dc = 256, 5120
    A, Dskip, dt_bias, h0 = inputs.decode_params(batch, Dc)
    r = np.random.default_rng(5)
    bsel = np.sort(np.concatenate([[0, batch - 1], r.choice(np.arange(1, batch - 1), 14, replace=False)]))
    dsel = np.sort(np.concatenate([[0, 63, 64, Dc - 1], r.choice(np.arange(65, Dc - 1), 252, replace=False)]))
    h = f32dev(h0)
    hs = h0[bsel][:, dsel].astype(np.float64)             # oracle state of the sample
    ib, idd = torch.from_numpy(bsel).cuda(), torch.from_numpy(dsel).cuda()
    tA, tD, tb = f32dev(A), f32dev(Dskip), f32dev(dt_bias)
    worst_y = worst_h = 0.0
    for step in range(1000):
        tok = inputs.decode_token(step, batch, Dc)
        y = binding.state_update(h, dev(tok.x, "bf16"), dev(tok.delta, "bf16"), tA, dev(tok.B, "bf16"),
                                 dev(tok.C, "bf16"), tD, tb, z=dev(tok.z, "bf16"))
        yg = host64(y.index_select(0, ib).index_select(1, idd))
        hg = host64(h.index_select(0, ib).index_select(1, idd))
        sub = lambda a: a[bsel][:, dsel]
        yo, hs = oracle.state_update(hs, sub(tok.x), sub(tok.delta), A[dsel], tok.B[bsel], tok.C[bsel],
                                     Dskip[dsel], dt_bias[dsel], z=sub(tok.z), io="bf16")
        ey = np.max(np.abs(yg - yo)) / np.max(np.abs(yo))
        eh = np.max(np.abs(hg - hs)) / np.max(np.abs(hs))
        worst_y, worst_h = max(worst_y, ey), max(worst_h, eh)
        assert ey <= TOL["bf16"], f"step {step}: y err {ey:.3e}"
        assert eh <= TOL["bf16"], f"step {step}: h err {eh:.3e}"
        if step % 100 == 0 or step == 999:
            log(f"decode step {step}: y err {ey:.3e} h err {eh:.3e} (worst so far {worst_y:.3e}, {worst_h:.3e})")
