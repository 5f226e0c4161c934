"""Float64 CPU oracle for the selective scan (S6). Test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never does.
"""
from .s6 import conv_scan_fwd, conv_silu, conv_state_update, decode, recurrence, scan_bwd, scan_fwd, silu, softplus, state_update  # noqa: F401
from .ssd import ssd_fwd  # noqa: F401
