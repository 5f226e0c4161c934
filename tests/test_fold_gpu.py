"""The chunk-carry combine at its structural boundaries (needs an MI355X).

The combine folds each wavefront's segment of carries, scans the segment
aggregates across lanes, and re-folds; a workgroup has 1, 2, 4 or 8
wavefronts (one while 32 carries or fewer, then enough for at most 32 carries
each), and takes the carries in rounds of up to 256.  These cases put the
carry count on each side of every change,
forward (folded from h0) and backward (the adjoint folded in reverse from
dh_last), and compare with the float64 oracle.  Workgroups are placed on the
XCD that wrote their carries when the channel blocks spread evenly over the
XCDs: the 8 x 300-channel cases take that placement with partial groups.
"""
import pytest

from gpu_util import TOL, assert_close, assert_grads_close, gpu_bwd, gpu_scan, host64, log, oracle_bwd, oracle_scan
from selective_state_space_39_amd import binding, inputs

pytestmark = pytest.mark.gpu

CHUNK = 32


def _length(ncar):
    """A sequence of ncar + 1 chunks of 32 tokens, the last one ragged (27 tokens)."""
    return (ncar + 1) * CHUNK - 5


@pytest.mark.parametrize("ncar", [1, 9, 31, 32, 33, 64, 65, 128, 129, 256, 257, 511, 512, 513, 700])
def test_forward_combine(ncar):
    L = _length(ncar)
    assert binding.plan(1, L, 70, binding.SSM_F32, CHUNK) == (CHUNK, ncar + 1)
    # 70 channels: a full and a partial 64-channel group
    s = inputs.make_scan_inputs(1, L, 70, io="f32", seed=(39, 7000 + ncar), with_h0=True)
    log(f"forward combine: {ncar} carries, L {L}")
    y, h = gpu_scan(s, chunk_len=CHUNK, h0=s.h0)
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(y), ry, TOL["f32"], f"{ncar} carries y")
    assert_close(host64(h), rh, TOL["f32"], f"{ncar} carries h_L")


@pytest.mark.parametrize("ncar", [20, 100])
def test_forward_combine_xcd_placed(ncar):
    """8 batch rows of 300 channels: 16 channel blocks, a multiple of the 8
    XCDs, so each group is combined on the XCD its carries came from; the
    second block of a row holds one partial 64-channel group and three empty
    ones."""
    L = _length(ncar)
    s = inputs.make_scan_inputs(8, L, 300, io="f32", seed=(39, 7200 + ncar), with_h0=True)
    log(f"forward combine, 8 x 300 channels: {ncar} carries, L {L}")
    y, h = gpu_scan(s, chunk_len=CHUNK, h0=s.h0)
    ry, rh = oracle_scan(s, h0=s.h0)
    assert_close(host64(y), ry, TOL["f32"], f"8 x 300, {ncar} carries y")
    assert_close(host64(h), rh, TOL["f32"], f"8 x 300, {ncar} carries h_L")


@pytest.mark.parametrize("ncar", [20, 100])
def test_backward_combine_xcd_placed(ncar):
    L = _length(ncar)
    s = inputs.make_scan_inputs(8, L, 300, io="f32", seed=(39, 7300 + ncar), with_h0=True, A_random=True)
    go = inputs.make_grad_outputs(8, L, 300, io="f32", seed=(39, 7300 + ncar), with_dh_last=True)
    log(f"backward combine, 8 x 300 channels: {ncar} carries, L {L}")
    g = gpu_bwd(s, go, chunk_len=CHUNK)
    ref = oracle_bwd(s, go)
    assert_grads_close(g, ref, TOL["f32"], f"bwd 8 x 300, {ncar} carries")


@pytest.mark.parametrize("ncar", [31, 129, 513])
def test_backward_combine(ncar):
    L = _length(ncar)
    s = inputs.make_scan_inputs(1, L, 33, io="f32", seed=(39, 7100 + ncar), with_h0=True, A_random=True)
    go = inputs.make_grad_outputs(1, L, 33, io="f32", seed=(39, 7100 + ncar), with_dh_last=True)
    log(f"backward combine: {ncar} carries, L {L}")
    g = gpu_bwd(s, go, chunk_len=CHUNK)
    ref = oracle_bwd(s, go)
    assert_grads_close(g, ref, TOL["f32"], f"bwd {ncar} carries")
