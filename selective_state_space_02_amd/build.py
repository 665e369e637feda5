"""Build libssm_scan.so in-tree with hipcc for gfx950.

``python -m selective_state_space_02_amd.build`` (or __graft_entry__.build()).
All device code is compiled with packed-FP32 instruction selection disabled
(``-packed-fp32-ops``); plain FP32 VALU ops already issue at full rate on gfx950.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssm_scan.so")
RATES_LIB = os.path.join(PKG, "libssm_rates.so")
SOURCES = [os.path.join(CSRC, "scan_api.cpp"), os.path.join(CSRC, "scan_kernels.hip"),
           os.path.join(CSRC, "update_kernels.hip"), os.path.join(CSRC, "ssd_kernels.hip"),
           os.path.join(CSRC, "scratch.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unknown-pragmas",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = ("not a recognized feature", "packed-fp32-ops")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile the host API (plain C++, -x c++) and the kernels (HIP), link one .so.

    scan_kernels.hip is compiled twice, once per discretization (-DSSM_ZOH=0/1); the
    device compilations run in parallel.
    """
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    api_o = os.path.join(objdir, "scan_api.o")
    jobs = [([HIPCC, *hipcc_flags(), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c", "-o",
              api_o, SOURCES[0]], api_o)]
    for src in SOURCES[1:]:
        stem = os.path.splitext(os.path.basename(src))[0]
        variants = [("_delta_b", ["-DSSM_ZOH=0"]), ("_zoh", ["-DSSM_ZOH=1"])] if stem == "scan_kernels" else [("", [])]
        for suffix, defs in variants:
            obj = os.path.join(objdir, stem + suffix + ".o")
            jobs.append(([HIPCC, *hipcc_flags(), *defs, "-x", "hip", "-c", "-o", obj, src], obj))
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    objs = [o for _, o in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    build_rates(verbose)
    return LIB


def build_rates(verbose: bool = False) -> str:
    """The issue-rate measurements behind the rooflines (bench.py --valu-rates), a library of
    their own: nothing in the scan library depends on them."""
    tmp = RATES_LIB + ".tmp"
    _run([HIPCC, *hipcc_flags(), "-shared", "-o", tmp, os.path.join(CSRC, "valu_rates.hip")], verbose)
    os.replace(tmp, RATES_LIB)
    return RATES_LIB


if __name__ == "__main__":
    print(build(verbose=True))
