"""MI355X-native selective state-space scan (S6) forward.

The compute path is the C-ABI library ``libssm_scan.so`` (hand-written HIP
kernels for gfx950, declared in include/ssm_scan.h).  ``scan.ssm_scan_fwd``
is a thin ctypes binding over it; PyTorch only owns device memory and streams.
Importing this package loads nothing: the library is opened on first use and
the call fails loudly if it is missing.
"""

__all__ = ["ssm_scan", "ssm_scan_fwd", "ssm_conv_scan_fwd", "ssm_state_update", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import scan
        return getattr(scan, name)
    raise AttributeError(name)
