"""The float64 oracle against its pins (closed forms, limits, brute force)."""
import numpy as np
import pytest

import oracle
import oracle.s6 as s6
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(s6)


def test_decode_bf16_all_patterns():
    """The oracle's bf16 decode agrees with torch's bfloat16 widening on all 65536 patterns."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_decode_rejects_wrong_storage():
    with pytest.raises(TypeError):
        oracle.decode(np.zeros(3, np.float32), "bf16")
    with pytest.raises(TypeError):
        oracle.decode(np.zeros(3, np.uint16), "f32")


def test_io_decoding_matches_numbers():
    """scan_fwd on bf16 storage equals scan_fwd on the decoded numbers."""
    from selective_state_space_39_amd import inputs
    s = inputs.make_scan_inputs(2, 19, 5, io="bf16", seed=(39, 900), with_h0=True)
    dec = lambda a: inputs.bf16_to_f32(a).astype(np.float64)
    y1, h1 = oracle.scan_fwd(s.x, s.delta, s.A, s.B, s.C, s.Dskip, s.dt_bias, z=s.z, h0=s.h0, io="bf16")
    y2, h2 = oracle.scan_fwd(dec(s.x), dec(s.delta), s.A, dec(s.B), dec(s.C), s.Dskip, s.dt_bias,
                             z=dec(s.z), h0=s.h0)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)
