"""The largest shapes the library accepts along its 32-bit offset limits (needs an MI355X).

Kernels address a scan chunk's rows, and one SSD batch row's x, z and y, through
buffer resources with 32-bit byte offsets; the host rejects any shape beyond
that.  These cases sit at the limit itself, with tensors well past 4 GiB, so a
64-bit base computed wrongly anywhere (a second batch row, a last chunk) shows
up.  Inputs are a small seeded problem tiled along the channels (or heads):
every tile must come out bit-identical to the first, and the first and last
tiles must match the float64 oracle of the small problem.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, assert_close, host64, log
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu

BASE = 64         # channels of the seeded problem that is tiled


def _tiled_dev(a, reps, axis):
    """Tile a host array along one axis and upload it (host copy dropped at once)."""
    shape = [1] * a.ndim
    shape[axis] = reps
    t = torch.from_numpy(np.tile(a, shape)).cuda()
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


def test_scan_chunk_at_the_32bit_offset_limit():
    """fp32 io, D = 16384: the longest chunk allowed, 32736 tokens (32736 x 16384 x 4 B just under 2 GiB), two
    batch rows of 33736 tokens each (the second row's last chunk starts 6.6 GB into each tensor)."""
    import oracle
    batch, L, D = 2, 33736, 16384
    cl = (2 ** 31 - 1) // (4 * D) // 32 * 32
    assert cl == 32736 and binding.plan(batch, L, D, binding.SSM_F32, cl) == (cl, 2)
    with pytest.raises(binding.SSMError):                # one more 32-token step is refused
        binding.plan(batch, L, D, binding.SSM_F32, cl + 32)
    s = inputs.make_scan_inputs(batch, L, BASE, io="f32", seed=(39, 2200), with_h0=True)
    reps = D // BASE
    log(f"scan {batch} x {L} x {D} fp32, chunk {cl}: {batch * L * D * 4 / 2 ** 30:.1f} GiB per tensor")
    x, dl, z = (_tiled_dev(a, reps, 2) for a in (s.x, s.delta, s.z))
    A, Dk, bias = (_tiled_dev(a, reps, 0) for a in (s.A, s.Dskip, s.dt_bias))
    h0 = _tiled_dev(s.h0, reps, 1)
    y, h = binding.scan_fwd(x, dl, A, _tiled_dev(s.B, 1, 0), _tiled_dev(s.C, 1, 0), Dk, bias, z=z, h0=h0,
                            chunk_len=cl)
    torch.cuda.synchronize()
    del x, dl, z
    yt, ht = y.view(batch, L, reps, BASE), h.view(batch, reps, BASE, 16)
    assert bool((yt == yt[:, :, :1]).all()), "a channel tile of y differs from the first"
    assert bool((ht == ht[:, :1]).all()), "a channel tile of h_L differs from the first"
    ry, rh = oracle.scan_fwd(s.x, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, z=s.z, h0=s.h0, io=s.io)
    for k in (0, reps - 1):
        assert_close(host64(yt[:, :, k].contiguous()), ry, TOL["f32"], f"y, tile {k}")
        assert_close(host64(ht[:, k].contiguous()), rh, TOL["f32"], f"h_L, tile {k}")



def test_conv_scan_chunk_at_the_32bit_offset_limit():
    """The scan fed by the width-4 convolution at the same limit: the second chunk's window starts from the
    three rows before it, 2 GiB into each batch row."""
    import oracle
    batch, L, D, K = 2, 33736, 16384, 4
    cl = (2 ** 31 - 1) // (4 * D) // 32 * 32
    s = inputs.make_scan_inputs(batch, L, BASE, io="f32", seed=(39, 2230), with_h0=True)
    cp = inputs.make_conv_params(batch, BASE, K, io="f32", seed=(39, 2230), with_init=True)
    reps = D // BASE
    log(f"conv scan {batch} x {L} x {D} fp32, K {K}, chunk {cl}")
    xin, dl, z = (_tiled_dev(a, reps, 2) for a in (s.x, s.delta, s.z))
    A, Dk, bias, cb = (_tiled_dev(a, reps, 0) for a in (s.A, s.Dskip, s.dt_bias, cp.b))
    cw = _tiled_dev(cp.w, reps, 0)
    h0, init = _tiled_dev(s.h0, reps, 1), _tiled_dev(cp.init, reps, 2)
    y, h, last = binding.conv_scan_fwd(xin, cw, cb, dl, A, _tiled_dev(s.B, 1, 0), _tiled_dev(s.C, 1, 0), Dk, bias,
                                       z=z, h0=h0, conv_init=init, chunk_len=cl, return_conv_last=True)
    torch.cuda.synchronize()
    assert torch.equal(last, xin[:, L - (K - 1):]), "conv_last is not the last K - 1 inputs"
    del xin, dl, z
    yt, ht = y.view(batch, L, reps, BASE), h.view(batch, reps, BASE, 16)
    assert bool((yt == yt[:, :, :1]).all()), "a channel tile of y differs from the first"
    assert bool((ht == ht[:, :1]).all()), "a channel tile of h_L differs from the first"
    ry, rh = oracle.conv_scan_fwd(s.x, cp.w, cp.b, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, z=s.z, h0=s.h0,
                                  conv_init=cp.init, io=s.io)
    for k in (0, reps - 1):
        assert_close(host64(yt[:, :, k].contiguous()), ry, TOL["f32"], f"conv y, tile {k}")
        assert_close(host64(ht[:, k].contiguous()), rh, TOL["f32"], f"conv h_L, tile {k}")

def test_ssd_batch_row_at_the_32bit_offset_limit():
    """SSD layer, 80 heads, N = 128, L = 209715: one batch row's x, z and y are 2 147 481 600 bytes each, the
    largest L the library accepts at 80 heads (one more token is refused)."""
    import oracle
    batch, L, H, N = 1, 209715, 80, 128
    assert L * H * 64 * 2 <= 2 ** 31 - 1 < (L + 1) * H * 64 * 2
    assert binding.lib().ssm_ssd_fwd_workspace_bytes(batch, L + 1, H, 64, N, binding.SSM_BF16) == -2
    q = inputs.make_ssd_inputs(batch, L, 1, N=N, seed=(39, 2210), with_h0=True)
    log(f"ssd {batch} x {L} x {H} heads, N {N}: {batch * L * H * 64 * 2 / 2 ** 30:.2f} GiB per tensor")
    x, z = (_tiled_dev(a, H, 2) for a in (q.x, q.z))
    dl = _tiled_dev(q.delta, H, 2)
    A, Dk, bias = (_tiled_dev(a, H, 0) for a in (q.A, q.Dskip, q.dt_bias))
    h0 = _tiled_dev(q.h0, H, 1)
    B, C = (torch.from_numpy(a).cuda().view(torch.bfloat16) for a in (q.B, q.C))
    y, h = binding.ssd_fwd(x, dl, A, B, C, Dk, bias, z=z, h0=h0)
    torch.cuda.synchronize()
    del x, z
    assert bool((y == y[:, :, :1]).all()), "a head of y differs from the first"
    assert bool((h == h[:, :1]).all()), "a head of h_L differs from the first"
    ry, rh = oracle.ssd_fwd(q.x, q.delta, q.A, q.B, q.C, q.Dskip, q.dt_bias, z=q.z, h0=q.h0, io=q.io)
    for k in (0, H - 1):
        assert_close(host64(y[:, :, k:k + 1].contiguous()), ry, TOL["bf16"], f"ssd y, head {k}")
        assert_close(host64(h[:, k:k + 1].contiguous()), rh, TOL["bf16"], f"ssd h_L, head {k}")


def test_backward_chunk_at_the_32bit_offset_limit():
    """The backward with the same longest fp32 chunk (32736 tokens of 16384 channels, two batch rows, 36 GiB of
    sub-chunk checkpoints in the workspace).  Per-channel gradients are bit-equal across tiles; dB and dC sum
    over all 16384 channels, i.e. 256 times the small problem's sums."""
    import oracle
    batch, L, D = 2, 33736, 16384
    cl = (2 ** 31 - 1) // (4 * D) // 32 * 32
    assert binding.bwd_plan(batch, L, D, binding.SSM_F32, cl) == (cl, 2)
    s = inputs.make_scan_inputs(batch, L, BASE, io="f32", seed=(39, 2220), with_h0=True, A_random=True)
    go = inputs.make_grad_outputs(batch, L, BASE, io="f32", seed=(39, 2220), with_dh_last=True)
    reps = D // BASE
    log(f"backward {batch} x {L} x {D} fp32, chunk {cl}: workspace "
        f"{binding.lib().ssm_scan_bwd_workspace_bytes(batch, L, D, 16, binding.SSM_F32, cl) / 2 ** 30:.1f} GiB")
    x, dl, z, dout = (_tiled_dev(a, reps, 2) for a in (s.x, s.delta, s.z, go.dout))
    A, Dk, bias = (_tiled_dev(a, reps, 0) for a in (s.A, s.Dskip, s.dt_bias))
    h0, dh_last = (_tiled_dev(a, reps, 1) for a in (s.h0, go.dh_last))
    g = binding.scan_bwd(x, dl, A, _tiled_dev(s.B, 1, 0), _tiled_dev(s.C, 1, 0), Dk, bias, dout, z=z, h0=h0,
                         dh_last=dh_last, chunk_len=cl)
    torch.cuda.synchronize()
    del x, dl, z, dout
    ref = oracle.scan_bwd(s.x, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, go.dout, z=s.z, h0=s.h0,
                          dh_last=go.dh_last, io=s.io)
    per_element = (batch, L, reps, BASE)                # tile axis 2
    for k, shape, ax in (("x", per_element, 2), ("delta", per_element, 2), ("z", per_element, 2),
                         ("h0", (batch, reps, BASE, 16), 1)):
        t = g[k].view(shape)
        assert bool((t == t.narrow(ax, 0, 1)).all()), f"a channel tile of d{k} differs from the first"
        for j in (0, reps - 1):
            assert_close(host64(t.select(ax, j).contiguous()), ref[k], TOL["f32"], f"d{k}, tile {j}")
    for k, n in (("A", 16), ("Dskip", 0), ("dt_bias", 0)):
        t = g[k].view(reps, BASE, n) if n else g[k].view(reps, BASE)
        assert bool((t == t[:1]).all()), f"a channel tile of d{k} differs from the first"
        for j in (0, reps - 1):
            assert_close(host64(t[j].contiguous()), ref[k], TOL["f32"], f"d{k}, tile {j}")
    for k in ("B", "C"):
        assert_close(host64(g[k]) / reps, ref[k], TOL["f32"], f"d{k} / {reps}")
