"""C-ABI boundary tests that need no GPU: the library loads, exports every
function include/ssm_scan.h declares, and rejects bad arguments with the
documented code before making any HIP call.

Only invalid argument sets are passed here (fake but aligned addresses), so
nothing can reach a kernel launch.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_02_amd import scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(ssm_[a-z_]+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = scan.load_library()
    names = header_functions()
    assert set(names) == set(scan.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ssm_scan_version() >= 100


def test_header_error_codes_match_binding():
    src = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"#define (SSM_(?:OK|ERR_[A-Z_]+))\s+(-?\d+)", src))
    for k, v in codes.items():
        assert getattr(scan, k) == v, k
    for v in codes.values():
        assert scan.strerror(v)
    assert scan.strerror(12345) == "unknown error code"


# fake, 16-byte aligned, non-overlapping addresses (1 MiB apart); never dereferenced
BASE = 1 << 40
P = {k: BASE + i * (1 << 30) for i, k in enumerate(
    ["u", "delta", "A", "B", "C", "D", "z", "bias", "h0", "y", "h_last", "ws"])}


def dims(**kw):
    d = dict(layout="bdl", io_dtype="bf16", batch=2, seqlen=64, dim=128, dstate=16)
    d.update(kw)
    return scan.make_dims(**d)


def call(dm, **over):
    a = dict(P)
    a.update(over)
    return scan.call_raw(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], True, a["h0"],
                         a["y"], a["h_last"], dm)


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "y"])
def test_null_required_pointer(name):
    assert call(dims(), **{name: None}) == scan.SSM_ERR_NULL_ARG


def test_null_dims():
    lib = scan.load_library()
    rc = lib.ssm_scan_fwd(P["u"], P["delta"], P["A"], P["B"], P["C"], None, None, None, 1, None, P["y"], None,
                          None, None)
    assert rc == scan.SSM_ERR_NULL_ARG


@pytest.mark.parametrize("kw", [dict(batch=0), dict(seqlen=0), dict(dim=0), dict(dstate=0), dict(ngroups=0),
                                dict(dim=100, ngroups=3), dict(seqlen=-5), dict(batch=70000)])
def test_bad_dims_bdl(kw):
    assert call(dims(**kw)) == scan.SSM_ERR_BAD_DIMS


@pytest.mark.parametrize("kw", [dict(nheads=3, headdim=64), dict(nheads=0, headdim=64), dict(nheads=2, headdim=0),
                                dict(nheads=2, headdim=64, ngroups=3),
                                dict(nheads=1 << 62, headdim=1 << 62), dict(nheads=-(1 << 62), headdim=-2)])
def test_bad_dims_blhp(kw):
    d = dict(layout="blhp", dim=128)
    d.update(kw)
    assert call(dims(**d)) == scan.SSM_ERR_BAD_DIMS


def test_unsupported():
    d = dims(dstate=257)
    assert call(d) == scan.SSM_ERR_UNSUPPORTED
    d = dims()
    d.layout = 7
    assert call(d) == scan.SSM_ERR_UNSUPPORTED
    d = dims()
    d.io_dtype = 3
    assert call(d) == scan.SSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "D", "z", "bias", "h0", "y", "h_last"])
def test_misaligned(name):
    assert call(dims(), **{name: P[name] + 4}) == scan.SSM_ERR_ALIGN


@pytest.mark.parametrize("out,inp", [("y", "u"), ("y", "z"), ("y", "B"), ("h_last", "h0"), ("h_last", "A"),
                                     ("y", "h_last")])
def test_alias(out, inp):
    assert call(dims(), **{out: P[inp] + 16}) == scan.SSM_ERR_ALIAS


def test_workspace_too_small():
    d = dims(layout="bdl", batch=1, seqlen=8192, dim=64, dstate=16)   # one row block: time is segmented
    need = scan.workspace_size(d)
    assert need > 0
    d.workspace = P["ws"]
    d.workspace_bytes = need - 1
    assert call(d) == scan.SSM_ERR_WORKSPACE


def bc_tile_bytes(batch, seqlen, npad, groups=1):
    """fp32 B/C tiles of the row-group kernel: 32-step blocks x (B and C) x padded states."""
    n = batch * groups * ((seqlen + 31) // 32) * 32 * 2 * npad * 4
    return (n + 255) // 256 * 256


def test_workspace_size_and_plan():
    d = dims(batch=4, seqlen=2048, dim=5120, dstate=16)               # 320 row blocks: no segments
    assert scan.workspace_size(d) == bc_tile_bytes(4, 2048, 16)
    assert "seg_len=2048" in scan.describe(d)
    txt = scan.describe(d)
    assert "kernel=rowgroup_mixed4" in txt and "layout=bdl" in txt and "grid=(64,4,1)" in txt
    d2 = dims(batch=8, seqlen=2048, dim=1536, dstate=16)              # 256 workgroups of 48 channels
    assert "kernel=rowgroup_mixed48" in scan.describe(d2) and "grid=(32,8,1)" in scan.describe(d2)
    d32 = dims(batch=4, seqlen=2048, dim=5120, dstate=32)             # 32 states: plain
    assert "kernel=rowgroup " in scan.describe(d32)
    d4 = dims(batch=1, seqlen=131072, dim=2560, dstate=16)            # 32 workgroups: 8 time segments
    assert scan.workspace_size(d4) == bc_tile_bytes(1, 131072, 16) + 2 * 7 * 1 * 16 * 2560 * 4
    assert "kernel=rowgroup_mixed4" in scan.describe(d4) and "grid=(32,1,8)" in scan.describe(d4)
    d5 = scan.make_dims("blhp", "bf16", 2, 8192, 5120, 128, nheads=80, headdim=64, ngroups=1)
    # 320 workgroups: 3 time segments of 43 chunks; two aggregates of (decay per head, state)
    assert "kernel=ssd" in scan.describe(d5) and "grid=(2,2,3)" in scan.describe(d5)
    assert "seg_len=2752" in scan.describe(d5)
    assert scan.workspace_size(d5) == 1280 + 2 * 2 * 5120 * 128 * 4
    d5f = scan.make_dims("blhp", "f32", 2, 8192, 5120, 128, nheads=80, headdim=64, ngroups=1)
    assert "kernel=workgroup" in scan.describe(d5f) and "NS=16" in scan.describe(d5f)
    d5n = scan.make_dims("blhp", "bf16", 2, 8192, 5120, 100, nheads=80, headdim=64, ngroups=1)
    assert "kernel=workgroup" in scan.describe(d5n)
    bad = dims(dim=0)
    assert scan.workspace_size(bad) == 0
    with pytest.raises(ValueError):
        scan.describe(bad)


def test_segment_override_env(monkeypatch):
    d = dims(batch=4, seqlen=2048, dim=5120, dstate=16)
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "4")
    assert scan.workspace_size(d) == bc_tile_bytes(4, 2048, 16) + 2 * 3 * 4 * 16 * 5120 * 4
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "1")
    assert scan.workspace_size(d) == bc_tile_bytes(4, 2048, 16)       # one segment: the mixed launch
    d = scan.make_dims("blhp", "bf16", 2, 8192, 5120, 128, nheads=80, headdim=64, ngroups=1)
    assert scan.workspace_size(d) == 0                                 # chunked kernel, one segment


def test_binding_rejects_cpu_tensors():
    import torch
    u = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        scan.ssm_scan_fwd(u, u, torch.zeros(4, 2), torch.zeros(1, 1, 2, 8), torch.zeros(1, 1, 2, 8))


def call_update(dm, **over):
    a = dict(P)
    a.update(over)
    return scan.call_update_raw(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], True,
                                a["h0"], a["h_last"], a["y"], dm)


def test_update_rejects_bad_arguments():
    d1 = dims(seqlen=1)
    for name in ["u", "delta", "A", "B", "C", "y"]:
        assert call_update(d1, **{name: None}) == scan.SSM_ERR_NULL_ARG
    assert call_update(dims(seqlen=2)) == scan.SSM_ERR_BAD_DIMS
    assert call_update(dims(seqlen=1, dim=0)) == scan.SSM_ERR_BAD_DIMS
    assert call_update(dims(seqlen=1, dstate=300)) == scan.SSM_ERR_UNSUPPORTED
    assert call_update(d1, z=P["z"] + 4) == scan.SSM_ERR_ALIGN
    assert call_update(d1, y=P["u"]) == scan.SSM_ERR_ALIAS
    assert call_update(d1, h_last=P["h0"] + 16) == scan.SSM_ERR_ALIAS        # partial overlap of the state
    assert call_update(d1, h_last=P["A"]) == scan.SSM_ERR_ALIAS
    assert call_update(d1, y=P["h_last"]) == scan.SSM_ERR_ALIAS


def test_discretization_field():
    d = dims()
    assert "disc=delta_b" in scan.describe(d)
    dz = dims()
    dz.discretization = scan.SSM_DISC_ZOH
    assert "disc=zoh" in scan.describe(dz)
    assert scan.workspace_size(dz) == scan.workspace_size(d)
    bad = dims()
    bad.discretization = 2
    assert call(bad) == scan.SSM_ERR_UNSUPPORTED
    bad = dims(seqlen=1)
    bad.reserved = 1
    assert call_update(bad) == scan.SSM_ERR_UNSUPPORTED


def test_conv_scan_rejects_bad_arguments():
    def cv(**kw):
        a = dict(weight=P["A"], bias=P["D"], state_in=None, state_out=None, width=4, reserved=0)
        a.update(kw)
        return scan.Conv(a["weight"], a["bias"], a["state_in"], a["state_out"], a["width"], a["reserved"])

    def callc(conv, dm=None, **over):
        a = dict(P)
        a.update(over)
        return scan.call_conv_raw(a["u"], conv, a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], True,
                                  a["h0"], a["y"], a["h_last"], dm or dims())

    assert callc(None) == scan.SSM_ERR_NULL_ARG
    assert callc(cv(weight=None)) == scan.SSM_ERR_NULL_ARG
    assert callc(cv(width=0)) == scan.SSM_ERR_UNSUPPORTED
    assert callc(cv(width=5)) == scan.SSM_ERR_UNSUPPORTED
    assert callc(cv(reserved=1)) == scan.SSM_ERR_UNSUPPORTED
    assert callc(cv(), dims(dstate=64)) == scan.SSM_ERR_UNSUPPORTED                      # workgroup-kernel shape
    assert callc(cv(), scan.make_dims("blhp", "bf16", 2, 64, 128, 16, nheads=2, headdim=64)) == \
        scan.SSM_ERR_UNSUPPORTED                                                        # 16 states: scan kernel
    assert callc(cv(), scan.make_dims("blhp", "f32", 2, 64, 128, 64, nheads=2, headdim=64)) == \
        scan.SSM_ERR_UNSUPPORTED                                                        # float32: scan kernel
    assert callc(cv(), scan.make_dims("blhp", "bf16", 2, 64, 128, 64, nheads=16, headdim=8)) == \
        scan.SSM_ERR_UNSUPPORTED                                                        # head size not 16k
    assert callc(cv(state_in=P["ws"] + 4)) == scan.SSM_ERR_ALIGN
    assert callc(cv(state_out=P["u"])) == scan.SSM_ERR_ALIAS
    assert callc(cv(state_out=P["y"] + 16)) == scan.SSM_ERR_ALIAS
    assert callc(cv(state_in=P["ws"]), y=P["ws"] + 16) == scan.SSM_ERR_ALIAS


def test_ssd_override_env(monkeypatch):
    d5 = scan.make_dims("blhp", "bf16", 2, 8192, 5120, 128, nheads=80, headdim=64, ngroups=1)
    monkeypatch.setenv("SSM_SCAN_SSD", "0")
    assert "kernel=workgroup" in scan.describe(d5)


def test_mixed_launch_override_env(monkeypatch):
    """SSM_SCAN_MIXED forces the 16-state launch shape (0 plain, 1 80 channels, 48 channels);
    the workspace size follows the launch the plan picks."""
    d = dims(batch=4, seqlen=2048, dim=5120, dstate=16)
    ws = scan.workspace_size(d)
    monkeypatch.setenv("SSM_SCAN_MIXED", "0")
    assert "kernel=rowgroup " in scan.describe(d) and scan.workspace_size(d) == ws
    monkeypatch.setenv("SSM_SCAN_MIXED", "48")
    assert "kernel=rowgroup_mixed48" in scan.describe(d) and "grid=(107,4,1)" in scan.describe(d)
    monkeypatch.setenv("SSM_SCAN_MIXED", "1")
    d2 = dims(batch=8, seqlen=2048, dim=1536, dstate=16)
    assert "kernel=rowgroup_mixed4" in scan.describe(d2) and "grid=(20,8,1)" in scan.describe(d2)
    d4 = dims(batch=1, seqlen=131072, dim=2560, dstate=16)
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "3")
    assert "kernel=rowgroup_mixed4" in scan.describe(d4) and "grid=(32,1,3)" in scan.describe(d4)
    monkeypatch.setenv("SSM_SCAN_MIXED", "0")
    assert "kernel=rowgroup " in scan.describe(d4) and "grid=(80,1,3)" in scan.describe(d4)


def test_plan_segments_and_launch_choices(monkeypatch):
    """Launch and segment choices of the plan for a few shapes (host logic only)."""
    for k in ("SSM_SCAN_MIXED", "SSM_SCAN_SEGMENTS", "SSM_SCAN_SSD", "SSM_SSD_PS"):
        monkeypatch.delenv(k, raising=False)
    # the 48-channel launch keeps one segment unless segments are forced
    d = dims(batch=16, seqlen=2048, dim=768, dstate=16)
    assert "kernel=rowgroup_mixed48" in scan.describe(d) and "grid=(16,16,1)" in scan.describe(d)
    monkeypatch.setenv("SSM_SCAN_MIXED", "48")
    assert ",1)" in scan.describe(dims(batch=1, seqlen=131072, dim=2560, dstate=16)).split("grid=")[1].split()[0]
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "3")
    assert "grid=(54,1,3)" in scan.describe(dims(batch=1, seqlen=131072, dim=2560, dstate=16))
    monkeypatch.delenv("SSM_SCAN_MIXED")
    monkeypatch.delenv("SSM_SCAN_SEGMENTS")
    # chunked multi-head kernel: about three workgroups per CU, segments of at least two chunks
    mh = lambda B, L, H, P=64, N=128: scan.make_dims("blhp", "bf16", B, L, H * P, N, nheads=H, headdim=P, ngroups=1)
    assert "grid=(2,1,5)" in scan.describe(mh(1, 8192, 80))          # 160 workgroups -> 5 segments
    assert "grid=(2,8,1)" in scan.describe(mh(8, 8192, 80))          # 1280 workgroups: one segment
    assert "grid=(2,1,2)" in scan.describe(mh(1, 256, 8))            # 256 steps: at most 2 segments
    assert "grid=(2,1,1)" in scan.describe(mh(1, 100, 8))            # under two chunks: one segment
    d = mh(1, 8192, 80)
    nseg = 5
    assert scan.workspace_size(d) == (nseg - 1) * 80 * 4 + (nseg - 1) * 1 * 80 * 64 * 128 * 4   # decays, states
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "1")
    assert "grid=(2,1,1)" in scan.describe(d) and scan.workspace_size(d) == 0


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "ssm_scan.h"
int main(void) {
  ssm_dims_t d;
  char buf[256];
  memset(&d, 0, sizeof d);
  d.batch = 4; d.seqlen = 2048; d.dim = 5120; d.dstate = 16; d.ngroups = 1;
  d.layout = SSM_LAYOUT_BDL; d.io_dtype = SSM_BF16;
  if (ssm_scan_version() <= 0) return 1;
  if (ssm_scan_describe(&d, buf, sizeof buf) != SSM_OK || strncmp(buf, "kernel=", 7) != 0) return 2;
  if (ssm_scan_workspace_size(&d) == 0) return 3;           /* the B/C tiles */
  d.dim = 0;
  if (ssm_scan_describe(&d, buf, sizeof buf) != SSM_ERR_BAD_DIMS) return 4;
  if (strlen(ssm_strerror(SSM_ERR_BAD_DIMS)) == 0) return 5;
  if (ssm_scan_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, &d, NULL) != SSM_ERR_NULL_ARG)
    return 6;
  printf("ok %s\n", ssm_strerror(SSM_OK));
  return 0;
}
"""


def test_header_is_plain_c_and_a_c_program_links(tmp_path):
    """The boundary is a C ABI: the header compiles as strict C99 and C++, and a C program
    linked against the library calls its host-side entry points (no GPU needed)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host compiler")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    inc = os.path.join(ROOT, "include")
    r = subprocess.run(["g++", "-std=c++11", "-Wall", "-Werror", "-x", "c++", "-I", inc, "-c", str(src), "-o",
                        str(tmp_path / "caller_cxx.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    libdir = os.path.dirname(scan.library_path())
    exe = str(tmp_path / "caller")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc, str(src), "-L", libdir,
                        "-lssm_scan", f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr)


def test_noalloc_rejects_beyond_scratch_before_any_hip_call():
    """ssm_scan_fwd_noalloc validates like ssm_scan_fwd, then refuses a launch whose scratch
    exceeds the static device array, all before any HIP call (fake addresses here)."""
    cap = scan.scratch_capacity()
    assert cap == 32 << 20
    big = dims(batch=64, seqlen=131072, dim=16, dstate=16)
    assert scan.workspace_size(big) > cap
    a = dict(P)
    args = (a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], True, a["h0"], a["y"], a["h_last"])
    assert scan.call_noalloc_raw(*args, big) == scan.SSM_ERR_SCRATCH
    assert "static device scratch" in scan.strerror(scan.SSM_ERR_SCRATCH)
    # the ordinary argument checks come first
    assert scan.call_noalloc_raw(*args, dims(dim=0)) == scan.SSM_ERR_BAD_DIMS
    assert scan.call_noalloc_raw(None, *args[1:], dims()) == scan.SSM_ERR_NULL_ARG
    assert scan.call_noalloc_raw(*args[:9], a["u"] + 8, *args[10:], dims()) == scan.SSM_ERR_ALIGN


def test_hip_failures_surface_as_ssm_err_hip(monkeypatch):
    """On a host without a GPU the first HIP call of a valid call fails: the library returns
    SSM_ERR_HIP and ssm_strerror names the failing call with HIP's text, for the library-made
    workspace (hipMallocAsync), the allocation-free entry point's scratch lookup and a kernel
    launch.  The pointers are not device memory, so this runs only where no GPU is visible."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a host without a GPU (the arguments are not device pointers)")
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", "3")
    d = dims(batch=1, seqlen=4096)
    assert scan.workspace_size(d) > 0
    rc = call(d)                                                     # workspace NULL: the library allocates
    assert rc == scan.SSM_ERR_HIP and "hipMallocAsync" in scan.strerror(rc)
    rc = scan.call_noalloc_raw(P["u"], P["delta"], P["A"], P["B"], P["C"], P["D"], P["z"], P["bias"], True,
                               P["h0"], P["y"], P["h_last"], d)
    assert rc == scan.SSM_ERR_HIP and "hipGetDevice" in scan.strerror(rc)
    d.workspace, d.workspace_bytes = P["ws"], scan.workspace_size(d)
    rc = call(d)                                                     # caller workspace: the launch itself fails
    assert rc == scan.SSM_ERR_HIP and "kernel launch" in scan.strerror(rc)


def test_scratch_covers_every_workload():
    """The allocation-free entry point's static scratch holds the workspace of every workload
    the benchmark runs (plans are host-only: no GPU needed)."""
    from selective_state_space_02_amd.inputs import CONFIGS
    cap = scan.scratch_capacity()
    for name, c in CONFIGS.items():
        d = scan.make_dims(c["layout"], c["io_dtype"], c["batch"], c["seqlen"], c["dim"], c["dstate"],
                           c.get("nheads", 0), c.get("headdim", 0), c.get("ngroups", 1))
        for disc in ("delta_b", "zoh"):
            d.discretization = scan.DISCRETIZATIONS[disc]
            assert scan.workspace_size(d) <= cap, f"{name} ({disc}): {scan.workspace_size(d)} > {cap}"
