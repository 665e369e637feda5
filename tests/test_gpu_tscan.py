"""The time-parallel kernel (time spread over the lanes of a wave, in-row DPP scan of the
(decay, state) pairs, cross-row combine in LDS, register-cached second pass) against the
fp64 oracle: ragged lengths (not a multiple of the 256-step span or of 4), fewer than 16
states, groups, channel counts that leave idle waves, both storage types, optional
arguments, and one long sequence on sampled steps."""
import numpy as np
import pytest
import torch

from selective_state_space_02_amd import scan
from selective_state_space_02_amd.inputs import make_case
from test_gpu_parity import TOL, assert_close, gpu_run, long_sample_times, oracle_run

pytestmark = pytest.mark.gpu


def run_forced(c, monkeypatch, t_out=None):
    monkeypatch.setenv("SSM_SCAN_TSCAN", "1")
    monkeypatch.delenv("SSM_SCAN_SEGMENTS", raising=False)
    dims = scan.make_dims(c.layout, c.io_dtype, c.batch, c.seqlen, c.dim, c.dstate, ngroups=c.ngroups)
    assert scan.describe(dims).startswith("kernel=tscan"), scan.describe(dims)
    y, h = gpu_run(c)
    y_ref, h_ref = oracle_run(c, t_out=t_out)
    if t_out is not None:
        y = y.index_select(2, torch.as_tensor(t_out, device=y.device))
    tol = TOL[c.io_dtype]
    ey = assert_close(y, y_ref, tol, f"{c.name} y")
    eh = assert_close(h, h_ref, tol, f"{c.name} h_last")
    print(f"[gpu] tscan {c.name}: max scaled err y {ey:.2e} h {eh:.2e}", flush=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L,D,N,G", [(1, 4, 16, 1), (3, 5, 16, 1), (255, 8, 16, 1), (256, 4, 16, 1), (257, 7, 16, 1),
                                     (1000, 12, 13, 2), (777, 6, 1, 1), (2050, 16, 16, 4), (513, 3, 8, 1)])
def test_tscan_shapes(io, L, D, N, G, monkeypatch):
    c = make_case("tscan", layout="bdl", io_dtype=io, batch=2, seqlen=L, dim=D, dstate=N, ngroups=G,
                  seed=L * 13 + D * 7 + N, has_h0=True, A_kind="lognormal")
    run_forced(c, monkeypatch)


@pytest.mark.parametrize("opts", [dict(has_z=False), dict(has_D=False, has_bias=False), dict(delta_kind="wide"),
                                  dict(delta_kind="long"), dict(softplus=False, delta_kind="zero")])
def test_tscan_options(opts, monkeypatch):
    opts = dict(opts)
    softplus = opts.pop("softplus", True)
    c = make_case("tscan_opts", layout="bdl", io_dtype="bf16", batch=2, seqlen=900, dim=20, dstate=16, seed=5,
                  has_h0=True, A_kind="lognormal", **opts)
    c.softplus = softplus
    run_forced(c, monkeypatch)


def test_tscan_degenerate_decays(monkeypatch):
    for mode in ("zero", "huge_negative"):
        c = make_case("tscan_deg", layout="bdl", io_dtype="f32", batch=1, seqlen=600, dim=8, dstate=16, seed=9,
                      has_h0=True, A_kind="lognormal")
        A = c.tensors["A"]
        c.tensors["A"] = torch.zeros_like(A) if mode == "zero" else torch.full_like(A, -1e4)
        run_forced(c, monkeypatch)


def test_tscan_long_sequence_sampled(monkeypatch):
    c = make_case("tscan_long", layout="bdl", io_dtype="bf16", batch=1, seqlen=65536, dim=64, dstate=16, seed=17,
                  has_h0=True, has_z=False, A_kind="lognormal", delta_kind="long")
    run_forced(c, monkeypatch, t_out=long_sample_times(c.seqlen))
