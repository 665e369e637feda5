"""fp64 CPU oracle for the selective state-space scan (S6).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  It shares no
code with the HIP library (selective_state_space_02_amd/).

Two independent implementations of the same plain recurrence live here:
``scan_f64`` (C, ssm_oracle.c, threaded over rows) and ``scan_numpy_f64``
(numpy, vectorised over rows, loop over time).  Tests pin both against the
closed forms and special cases the pages fix.
"""
from .oracle import (  # noqa: F401
    LAYOUT_BDL,
    LAYOUT_BLHP,
    build,
    default_threads,
    lib_path,
    scan_f64,
    scan_numpy_f64,
    silu_f64,
    softplus_f64,
)
