"""GPU parity of the fused input stage (causal depthwise conv1d + SiLU, then the scan)
through ssm_conv_scan_fwd, against the oracle's conv_scan.  Widths 1..4, ragged
sequence lengths (element path), 16 and 32 states, forced time segments (the
segment's first block reads the 3 raw inputs before it), a carried conv state in
and out, the exact-hold discretization, a two-call continuation, and every
16-state launch (2, 4, 8 or 16 steps per lane take their 3 earlier raw inputs
from one or two lanes to the left, or from the carry of the previous block).  The multi-head layout (chunked kernel, bfloat16)
convolves each channel d = h*P + p along time: 32, 64 and 128 states, 16- and 32-position
slices, ragged last chunks, forced segments (a segment's first chunk reads the raw inputs
before it), the exact hold, and a two-call continuation.
Tolerances as for the scan: 1e-4 (float32) and 2e-2 (bfloat16) relative to 1 + |ref|.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_02_amd import scan
from selective_state_space_02_amd.inputs import make_case

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = torch.device("cuda:0")


def np_io(t, io):
    if t is None:
        return None
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if io == "bf16" else t.numpy()


def scaled_err(got, ref):
    got = got.double().cpu().numpy()
    assert np.isfinite(got).all()
    return float((np.abs(got - ref) / (1.0 + np.abs(ref))).max()) if ref.size else 0.0


def conv_params(Dm, K, Bsz, seed, with_state):
    g = torch.Generator().manual_seed(seed)
    w = (torch.randn(Dm, K, generator=g) * 0.5).contiguous()
    b = (torch.randn(Dm, generator=g) * 0.2).contiguous()
    st = torch.randn(Bsz, Dm, K - 1, generator=g).contiguous() if with_state else None
    return w, b, st


def run(c, w, b, st, disc="delta_b", h0=None):
    T = {k: (None if v is None else v.to(DEV)) for k, v in c.tensors.items()}
    h0 = T["h0"] if h0 is None else h0
    y, h, cs = scan.ssm_conv_scan_fwd(T["u"], w.to(DEV), None if b is None else b.to(DEV), T["delta"], T["A"],
                                      T["B"], T["C"], T["D"], T["z"], T["delta_bias"], c.softplus, h0,
                                      conv_state_in=None if st is None else st.to(DEV), want_conv_state=True,
                                      discretization=disc, layout=c.layout)
    torch.cuda.synchronize()
    return y, h, cs


def ref(c, w, b, st, disc="euler", h0=None):
    T = c.tensors
    f = lambda k: None if T[k] is None else T[k].numpy()
    return oracle.scan_f64(np_io(T["u"], c.io_dtype), np_io(T["delta"], c.io_dtype), f("A"),
                           np_io(T["B"], c.io_dtype), np_io(T["C"], c.io_dtype), f("D"), np_io(T["z"], c.io_dtype),
                           f("delta_bias"), c.softplus, f("h0") if h0 is None else h0, layout=c.layout,
                           io_dtype=c.io_dtype, ngroups=c.ngroups, discretization=disc, conv_w=w.numpy(),
                           conv_b=None if b is None else b.numpy(),
                           conv_state_in=None if st is None else st.numpy(), want_conv_state=True)


CASES = [
    ("bf16-K4", dict(io_dtype="bf16", batch=2, seqlen=320, dim=136, dstate=16), 4, True, None, "delta_b"),
    ("bf16-K3-nostate", dict(io_dtype="bf16", batch=1, seqlen=256, dim=64, dstate=16), 3, False, None, "delta_b"),
    ("f32-K2-ragged", dict(io_dtype="f32", batch=2, seqlen=97, dim=40, dstate=16), 2, True, None, "delta_b"),
    ("f32-K1", dict(io_dtype="f32", batch=1, seqlen=64, dim=24, dstate=5), 1, False, None, "delta_b"),
    ("f32-K4-N32", dict(io_dtype="f32", batch=1, seqlen=130, dim=64, dstate=32), 4, True, None, "delta_b"),
    ("f32-K4-segments", dict(io_dtype="f32", batch=1, seqlen=1100, dim=16, dstate=16), 4, True, "3", "delta_b"),
    ("bf16-K4-zoh", dict(io_dtype="bf16", batch=2, seqlen=200, dim=72, dstate=16), 4, True, None, "zoh"),
]


@pytest.mark.parametrize("name,kw,K,with_state,segs,disc", CASES, ids=[c[0] for c in CASES])
def test_conv_scan(name, kw, K, with_state, segs, disc, monkeypatch):
    if segs:
        monkeypatch.setenv("SSM_SCAN_SEGMENTS", segs)
    c = make_case(name, layout="bdl", seed=51, has_h0=True, A_kind="lognormal", **kw)
    w, b, st = conv_params(c.dim, K, c.batch, 52, with_state)
    print(f"[gpu] conv scan {name} K={K} state={with_state} segments={segs} disc={disc}", flush=True)
    y, h, cs = run(c, w, b, st, disc)
    y_ref, h_ref, cs_ref = ref(c, w, b, st, "zoh" if disc == "zoh" else "euler")
    tol = TOL[c.io_dtype]
    ey, eh = scaled_err(y, y_ref), scaled_err(h, h_ref)
    print(f"[gpu]   max scaled err y {ey:.2e} h {eh:.2e}", flush=True)
    assert ey <= tol and eh <= tol
    np.testing.assert_array_equal(cs.double().cpu().numpy(), cs_ref)


LAUNCHES = {"plain": {"SSM_SCAN_MIXED": "0"}, "mixed4": {"SSM_SCAN_MIXED": "1"}, "mixed48": {"SSM_SCAN_MIXED": "48"}}
LAUNCH_CASES = [
    ("bf16-K4", dict(io_dtype="bf16", batch=2, seqlen=320, dim=136, dstate=16), 4, True, None),
    ("f32-K3-ragged", dict(io_dtype="f32", batch=2, seqlen=97, dim=90, dstate=16), 3, True, None),
    ("f32-K4-segments", dict(io_dtype="f32", batch=1, seqlen=1100, dim=100, dstate=13), 4, True, "3"),
    ("bf16-K2-nostate", dict(io_dtype="bf16", batch=1, seqlen=200, dim=48, dstate=16), 2, False, None),
]


@pytest.mark.parametrize("launch", list(LAUNCHES))
@pytest.mark.parametrize("name,kw,K,with_state,segs", LAUNCH_CASES, ids=[c[0] for c in LAUNCH_CASES])
def test_conv_scan_launches(name, kw, K, with_state, segs, launch, monkeypatch):
    for k, v in LAUNCHES[launch].items():
        monkeypatch.setenv(k, v)
    if segs:
        monkeypatch.setenv("SSM_SCAN_SEGMENTS", segs)
    c = make_case(name, layout="bdl", seed=53, has_h0=True, A_kind="lognormal", **kw)
    w, b, st = conv_params(c.dim, K, c.batch, 54, with_state)
    print(f"[gpu] conv scan {name} launch={launch} K={K} segments={segs}", flush=True)
    y, h, cs = run(c, w, b, st)
    y_ref, h_ref, cs_ref = ref(c, w, b, st)
    tol = TOL[c.io_dtype]
    ey, eh = scaled_err(y, y_ref), scaled_err(h, h_ref)
    print(f"[gpu]   max scaled err y {ey:.2e} h {eh:.2e}", flush=True)
    assert ey <= tol and eh <= tol
    np.testing.assert_array_equal(cs.double().cpu().numpy(), cs_ref)


def test_conv_scan_continuation():
    c = make_case("cont", layout="bdl", io_dtype="f32", batch=2, seqlen=256, dim=48, dstate=16, seed=61,
                  has_h0=True, A_kind="lognormal")
    w, b, st = conv_params(c.dim, 4, c.batch, 62, True)
    print("[gpu] conv scan continuation", flush=True)
    y_ref, h_ref, cs_ref = ref(c, w, b, st)
    k = 100                                       # not a multiple of the 32-step block
    T = c.tensors
    part = lambda lo, hi: make_case("p", layout="bdl", io_dtype="f32", batch=2, seqlen=hi - lo, dim=48, dstate=16,
                                    seed=61, has_h0=True)
    c1, c2 = part(0, k), part(k, c.seqlen)
    for cc, lo, hi in ((c1, 0, k), (c2, k, c.seqlen)):
        for key in ("u", "delta", "z"):
            cc.tensors[key] = T[key][:, :, lo:hi].contiguous()
        for key in ("B", "C"):
            cc.tensors[key] = T[key][..., lo:hi].contiguous()
        for key in ("A", "D", "delta_bias"):
            cc.tensors[key] = T[key]
    c1.tensors["h0"] = T["h0"]
    y1, h1, cs1 = run(c1, w, b, st)
    c2.tensors["h0"] = None
    y2, h2, cs2 = run(c2, w, b, cs1.cpu(), h0=h1)
    y = torch.cat([y1, y2], dim=2)
    assert scaled_err(y, y_ref) <= TOL["f32"]
    assert scaled_err(h2, h_ref) <= TOL["f32"]
    np.testing.assert_array_equal(cs2.double().cpu().numpy(), cs_ref)


# ---------------------------------------------------------------------------
# Multi-head layout: the chunked kernel (bfloat16 storage, 32/64/128 states)
# ---------------------------------------------------------------------------

MH_CASES = [
    # name, shape, K, carried state, forced segments, discretization, forced 16-position slices
    ("mh-N128-K4", dict(batch=2, seqlen=200, nheads=4, headdim=64, dstate=128), 4, True, None, "delta_b", False),
    ("mh-N64-K3-nostate", dict(batch=1, seqlen=130, nheads=3, headdim=32, dstate=64), 3, False, None, "delta_b",
     False),
    ("mh-N32-P16-K2", dict(batch=2, seqlen=64, nheads=5, headdim=16, dstate=32), 2, True, None, "delta_b", False),
    ("mh-N128-K4-segments", dict(batch=1, seqlen=700, nheads=2, headdim=64, dstate=128), 4, True, "3", "delta_b",
     False),
    ("mh-N64-K4-zoh", dict(batch=2, seqlen=150, nheads=2, headdim=64, dstate=64), 4, True, None, "zoh", False),
    ("mh-N128-K1", dict(batch=1, seqlen=96, nheads=2, headdim=32, dstate=128), 1, False, None, "delta_b", False),
    ("mh-N128-K4-ps16", dict(batch=1, seqlen=190, nheads=2, headdim=64, dstate=128), 4, True, None, "delta_b", True),
    ("mh-N64-K4-short", dict(batch=2, seqlen=2, nheads=2, headdim=32, dstate=64), 4, True, None, "delta_b", False),
    ("mh-N128-K3-groups", dict(batch=1, seqlen=160, nheads=4, headdim=32, dstate=128, ngroups=2), 3, True, "2",
     "delta_b", False),
]


def mh_case(name, kw, seed):
    kw = dict(kw)
    kw["dim"] = kw["nheads"] * kw["headdim"]
    return make_case(name, layout="blhp", io_dtype="bf16", seed=seed, has_h0=True, A_kind="head_uniform", **kw)


@pytest.mark.parametrize("name,kw,K,with_state,segs,disc,ps16", MH_CASES, ids=[c[0] for c in MH_CASES])
def test_conv_scan_multihead(name, kw, K, with_state, segs, disc, ps16, monkeypatch):
    if segs:
        monkeypatch.setenv("SSM_SCAN_SEGMENTS", segs)
    if ps16:
        monkeypatch.setenv("SSM_SSD_PS", "16")
    c = mh_case(name, kw, 71)
    dims = scan.make_dims("blhp", "bf16", c.batch, c.seqlen, c.dim, c.dstate, c.nheads, c.headdim, c.ngroups)
    plan = scan.describe(dims)
    assert "kernel=ssd" in plan
    w, b, st = conv_params(c.dim, K, c.batch, 72, with_state)
    print(f"[gpu] conv scan {name} K={K} state={with_state} segments={segs} disc={disc} plan={plan}", flush=True)
    y, h, cs = run(c, w, b, st, disc)
    y_ref, h_ref, cs_ref = ref(c, w, b, st, "zoh" if disc == "zoh" else "euler")
    ey, eh = scaled_err(y, y_ref), scaled_err(h, h_ref)
    print(f"[gpu]   max scaled err y {ey:.2e} h {eh:.2e}", flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(cs.double().cpu().numpy(), cs_ref)


def test_conv_scan_multihead_continuation():
    c = mh_case("mh-cont", dict(batch=2, seqlen=256, nheads=2, headdim=64, dstate=128), 75)
    w, b, st = conv_params(c.dim, 4, c.batch, 76, True)
    print("[gpu] conv scan multi-head continuation", flush=True)
    y_ref, h_ref, cs_ref = ref(c, w, b, st)
    k = 100                                       # not a multiple of the 64-step chunk
    T = c.tensors
    parts = []
    for lo, hi in ((0, k), (k, c.seqlen)):
        cc = mh_case("p", dict(batch=2, seqlen=hi - lo, nheads=2, headdim=64, dstate=128), 75)
        for key in ("u", "delta", "z", "B", "C"):
            cc.tensors[key] = T[key][:, lo:hi].contiguous()
        for key in ("A", "D", "delta_bias"):
            cc.tensors[key] = T[key]
        parts.append(cc)
    parts[0].tensors["h0"] = T["h0"]
    y1, h1, cs1 = run(parts[0], w, b, st)
    parts[1].tensors["h0"] = None
    y2, h2, cs2 = run(parts[1], w, b, cs1.cpu(), h0=h1)
    y = torch.cat([y1, y2], dim=1)
    assert scaled_err(y, y_ref) <= TOL["bf16"]
    assert scaled_err(h2, h_ref) <= TOL["bf16"]
    np.testing.assert_array_equal(cs2.double().cpu().numpy(), cs_ref)


@pytest.mark.parametrize("name", ["mamba2p8b_layer", "mamba2_multihead"])
def test_workload_full_conv(name):
    """Both layer workloads at full size with the K = 4 input stage, in the launch and with the
    filters `bench.py --conv 4` times (same seeded recipe), against the oracle over every output."""
    from selective_state_space_02_amd.inputs import make_config
    c = make_config(name)
    gen = torch.Generator().manual_seed(20260999)
    w = (torch.randn(c.dim, 4, generator=gen) * 0.5).contiguous()
    b = (torch.randn(c.dim, generator=gen) * 0.2).contiguous()
    print(f"[gpu] conv scan full workload {name}", flush=True)
    y, h, cs = run(c, w, b, None)
    y_ref, h_ref, cs_ref = ref(c, w, b, None)
    ey, eh = scaled_err(y, y_ref), scaled_err(h, h_ref)
    print(f"[gpu]   max scaled err y {ey:.2e} h {eh:.2e}", flush=True)
    assert ey <= TOL[c.io_dtype] and eh <= TOL[c.io_dtype]
    np.testing.assert_array_equal(cs.double().cpu().numpy(), cs_ref)
