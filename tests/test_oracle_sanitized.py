"""The fp64 oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

An out-of-bounds read in the oracle would silently corrupt reference values, so
its C source is rebuilt with -fsanitize=address,undefined (gcc, host code) and,
in a child process that preloads the sanitizer runtimes, the oracle pins run
against that build, followed by a seeded sweep of small random cases over both
layouts, groups, gates, initial states, both discretizations, sampled outputs
and the input stage with and without a carried state.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SWEEP = r'''
import random, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import oracle.oracle as o
o._LIB = sys.argv[2]
import oracle
from selective_state_space_02_amd.inputs import make_case
o._load()
assert o._lib._name == sys.argv[2]
rng = random.Random(int(sys.argv[3]))
def npio(t, io):
    if t is None:
        return None
    t = t.contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if io == "bf16" else t.numpy()
for it in range(int(sys.argv[4])):
    layout, io = rng.choice(["bdl", "blhp"]), rng.choice(["f32", "bf16"])
    B, L, N, G = rng.choice([1, 2, 3]), rng.choice([1, 2, 5, 33, 100]), rng.choice([1, 3, 16, 33]), rng.choice([1, 2])
    if layout == "bdl":
        D, H, P = G * rng.choice([1, 3, 5]), 0, 0
    else:
        H, P = G * rng.choice([1, 2]), rng.choice([1, 4, 7])
        D = H * P
    c = make_case("s", layout=layout, io_dtype=io, batch=B, seqlen=L, dim=D, dstate=N, nheads=H, headdim=P, ngroups=G,
                  seed=it, A_kind="lognormal" if layout == "bdl" else "head_uniform", has_h0=rng.random() < 0.5,
                  has_z=rng.random() < 0.5, has_D=rng.random() < 0.5, has_bias=rng.random() < 0.5)
    T = c.tensors
    f = lambda k: None if T[k] is None else T[k].numpy()
    kw = dict(layout=layout, io_dtype=io, ngroups=G, discretization=rng.choice(["euler", "zoh"]))
    if layout == "bdl" and rng.random() < 0.3:
        K = rng.choice([1, 2, 3, 4])
        g = np.random.default_rng(it)
        kw["conv_w"] = g.standard_normal((D, K)).astype(np.float32)
        kw["conv_b"] = g.standard_normal(D).astype(np.float32) if rng.random() < 0.5 else None
        if K > 1 and rng.random() < 0.5:
            kw["conv_state_in"] = g.standard_normal((B, D, K - 1)).astype(np.float32)
        kw["want_conv_state"] = rng.random() < 0.5
    elif rng.random() < 0.3:
        kw["t_out"] = np.array(sorted(rng.sample(range(L), min(L, 3))), dtype=np.int64)
    r = oracle.scan_f64(npio(T["u"], io), npio(T["delta"], io), f("A"), npio(T["B"], io), npio(T["C"], io), f("D"),
                        npio(T["z"], io), f("delta_bias"), True, f("h0"), **kw)
    assert np.isfinite(r[0]).all()
print("ok")
'''


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_oracle(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if shutil.which("gcc") is None or asan is None or ubsan is None:
        pytest.skip("gcc or its sanitizer runtimes are missing")
    d = tmp_path_factory.mktemp("oracle_asan")
    lib = str(d / "libssm_oracle.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
                        os.path.join(ROOT, "oracle", "ssm_oracle.c"), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    pre = ":".join(x for x in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if x)   # the runtimes go first
    env = dict(os.environ, LD_PRELOAD=pre, ASAN_OPTIONS="detect_leaks=0")
    yield lib, env
    shutil.rmtree(str(d), ignore_errors=True)


def test_oracle_pins_under_sanitizers(sanitized_oracle):
    lib, env = sanitized_oracle
    code = (f"import sys, os; sys.path.insert(0, {ROOT!r}); import oracle.oracle as o; o._LIB = {lib!r}; "
            f"import pytest; rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(ROOT, 'tests', 'test_oracle_pins.py')!r}]); "
            f"assert o._lib is not None and o._lib._name == {lib!r}, 'the pins did not run the sanitized build'; "
            f"raise SystemExit(rc)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-3000:])


def test_oracle_sweep_under_sanitizers(sanitized_oracle):
    lib, env = sanitized_oracle
    r = subprocess.run([sys.executable, "-c", SWEEP, ROOT, lib, "11", "150"], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-3000:])
