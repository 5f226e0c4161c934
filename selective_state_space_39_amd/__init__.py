"""MI355X-native selective scan (S6): a HIP library for gfx950 behind a C ABI.

``scan_fwd`` and ``state_update`` (re-exported from the ctypes binding) are
the Python entry points; they marshal torch tensors into the C ABI and nothing
else. The binding loads ``libssm_scan.so`` on first use and raises if it is
missing or was built for another ABI version.
"""


def __getattr__(name):
    if name in ("scan_fwd", "state_update", "lib", "workspace_bytes", "abi_version", "SSMError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
