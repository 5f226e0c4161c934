"""Backward selective scan on the GPU against the float64 oracle (needs an MI355X).

Every gradient the library returns is compared element by element with
oracle.scan_bwd on the same seeded bits, at the io tolerance relative to the
largest reference value.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close, assert_grads_close, gpu_bwd, host64, log, oracle_bwd
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _case(batch, L, D, io, seed, gated=True, h0=True, dh=True, A_random=True):
    s = inputs.make_scan_inputs(batch, L, D, io=io, seed=(39, seed), gated=gated, with_h0=h0, A_random=A_random)
    go = inputs.make_grad_outputs(batch, L, D, io=io, seed=(39, seed), with_dh_last=dh)
    return s, go


@pytest.mark.parametrize("batch,L,D,io,gated,h0,dh,chunk", [
    (2, 300, 200, "bf16", True, True, True, 64),      # 5 chunks, ragged last (44 tokens)
    (1, 257, 130, "f32", False, False, False, 32),    # 9 chunks, last holds 1 token
    (3, 97, 65, "bf16", True, True, True, 32),        # odd D: 16-bit loads
    (2, 64, 64, "f32", True, True, True, 64),         # exactly one chunk
    (1, 1, 1, "bf16", True, False, True, 32),         # one token, one channel
    (2, 5, 3, "f32", False, True, False, 32),         # one ragged chunk: sub-chunks of 4 and 1
    (4, 512, 320, "bf16", True, True, True, 0),       # automatic plan
    (2, 1000, 96, "f32", True, True, True, 96),       # chunk not a power of two
])
def test_bwd_matches_oracle(batch, L, D, io, gated, h0, dh, chunk):
    s, go = _case(batch, L, D, io, 4000 + L + D, gated, h0, dh)
    log(f"bwd {batch}x{L}x{D} {io} gated={gated} h0={h0} dh={dh} plan {binding.bwd_plan(batch, L, D, 1, chunk)}")
    g = gpu_bwd(s, go, chunk_len=chunk, gated=gated, h0=h0)
    ref = oracle_bwd(s, go, gated=gated, h0=h0)
    assert_grads_close(g, ref, TOL[io], f"bwd {batch}x{L}x{D}")


@pytest.mark.parametrize("chunk", [32, 64, 160, 512])
def test_bwd_chunk_invariance(chunk):
    s, go = _case(2, 600, 192, "f32", 4100)
    g = gpu_bwd(s, go, chunk_len=chunk)
    ref = oracle_bwd(s, go)
    assert_grads_close(g, ref, TOL["f32"], f"bwd chunk {chunk}")


def test_bwd_deterministic():
    s, go = _case(4, 700, 320, "bf16", 4200)
    g1 = gpu_bwd(s, go, chunk_len=64)
    g2 = gpu_bwd(s, go, chunk_len=64)
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), f"d{k} differs between two identical calls"


def test_bwd_without_dh0():
    s, go = _case(2, 130, 64, "bf16", 4300)
    g = gpu_bwd(s, go, chunk_len=32, want_dh0=False)
    assert g["h0"] is None
    ref = oracle_bwd(s, go)
    ref["h0"] = None
    assert_grads_close(g, ref, TOL["bf16"], "bwd no dh0")


def test_bwd_full_size_mamba130m_layer():
    """The 130M-layer workload (8 x 2048 x 1536, bf16, S4D-real A) at the automatic plan."""
    s = inputs.make_workload("mamba-130m-layer")
    go = inputs.make_grad_outputs(8, 2048, 1536, io="bf16", seed=inputs.SCAN_WORKLOADS["mamba-130m-layer"]["seed"],
                                  with_dh_last=False)
    log(f"full-size bwd plan {binding.bwd_plan(8, 2048, 1536, 1, 0)}")
    g = gpu_bwd(s, go, h0=False)
    log("oracle (channel strips) ...")
    ref = oracle_bwd(s, go, h0=False, strip=192)
    assert_grads_close(g, ref, TOL["bf16"], "bwd 130M layer")


def test_bwd_full_size_mamba28b_layer_sampled_channels():
    """The 2.8B-layer workload (4 x 2048 x 5120, bf16) at the automatic plan: the per-channel
    gradients (dx, ddelta, dz, dA, dD, ddt_bias) of 64 sampled channels against the oracle run
    on those channels alone (dB and dC sum over every channel: the 130M-layer case checks them
    in full)."""
    name = "mamba-2.8b-layer"
    s = inputs.make_workload(name)
    go = inputs.make_grad_outputs(4, 2048, 5120, io="bf16", seed=inputs.SCAN_WORKLOADS[name]["seed"],
                                  with_dh_last=False)
    log(f"full-size bwd plan {binding.bwd_plan(4, 2048, 5120, 1, 0)}")
    g = gpu_bwd(s, go, h0=False)
    ch = np.unique(np.concatenate([[0, 63, 64, 5119], np.random.default_rng([39, 4400]).choice(5120, 60, replace=False)]))
    r = oracle.scan_bwd(s.x[:, :, ch], s.delta[:, :, ch], s.A[ch], s.B, s.C, s.Dskip[ch], s.dt_bias[ch],
                        go.dout[:, :, ch], z=s.z[:, :, ch], io="bf16")
    for k, axis in (("x", 2), ("delta", 2), ("z", 2), ("A", 0), ("Dskip", 0), ("dt_bias", 0)):
        v = host64(g[k])
        assert_close(v[:, :, ch] if axis == 2 else v[ch], r[k], TOL["bf16"], f"bwd 2.8B layer d{k} (sampled)")


def test_bwd_errors_raise_before_launch():
    s, go = _case(1, 64, 64, "bf16", 4400)
    with pytest.raises(binding.SSMError):
        gpu_bwd(s, go, chunk_len=48)


def test_bwd_outputs_overwrite_not_accumulate():
    """Preallocated gradient buffers holding garbage (NaN) are overwritten: the result equals a fresh call."""
    s, go = _case(2, 200, 96, "f32", 4500)
    fresh = gpu_bwd(s, go, chunk_len=64)
    shapes = {k: v for k, v in fresh.items() if v is not None}
    junk = {k: torch.full_like(v, float("nan")) for k, v in shapes.items()}
    from gpu_util import dev, f32dev
    io = s.io
    g = binding.scan_bwd(dev(s.x, io), dev(s.delta, io), f32dev(s.A), dev(s.B, io), dev(s.C, io),
                         f32dev(s.Dskip), f32dev(s.dt_bias), dev(go.dout, io), z=dev(s.z, io), h0=f32dev(s.h0),
                         dh_last=f32dev(go.dh_last), chunk_len=64, grads=junk)
    torch.cuda.synchronize()
    for k in shapes:
        assert g[k].data_ptr() == junk[k].data_ptr()
        assert torch.equal(g[k], fresh[k]), f"d{k} differs from a fresh call"
