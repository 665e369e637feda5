"""GPU parity over seeded random combinations of shape, options and launch.

Each case draws a layout, storage type, batch, length, channel count, state count (1 to
256), groups, optional arguments (gate, D, bias, initial state, no softplus), step-size regime
(small, wide, long-sequence, zero), the discretization, the fused input stage (with or without
a carried state, whose output is compared bit for bit), a single decode step (in place or not)
and a forced launch shape or time-segment count, then compares y and h_last with the fp64
oracle under the usual bounds (1e-4 float32, 2e-2
bfloat16, relative to 1 + |ref|).  Without softplus the step is delta itself (no bias), kept
positive.  The draws are fixed by the seed, so the cases are the same on every run.
"""
import os
import random

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_02_amd import scan
from selective_state_space_02_amd.inputs import make_case

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
ENV_KEYS = ("SSM_SCAN_MIXED", "SSM_SCAN_SSD", "SSM_SSD_PS", "SSM_SCAN_SEGMENTS")


def np_io(t, io):
    if t is None:
        return None
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if io == "bf16" else t.numpy()


def scaled_err(got, ref):
    got = got.double().cpu().numpy()
    if not np.isfinite(got).all():
        return float("inf")
    return float((np.abs(got - ref) / (1.0 + np.abs(ref))).max()) if ref.size else 0.0


def draw(rng, big, mh_conv=False):
    """mh_conv: only the multi-head layout through the input stage (bf16, the chunked kernel)."""
    layout = "blhp" if mh_conv else rng.choice(["bdl", "bdl", "bdl", "blhp"])
    io = "bf16" if mh_conv else rng.choice(["bf16", "f32"])
    B = rng.choice([1, 2, 3])
    L = rng.choice([1, 2, 7, 31, 32, 33, 64, 95, 128, 200, 257, 500, 1000] + ([2048, 3001, 4096] if big else []))
    conv, env = 0, {}
    if layout == "bdl":
        N = rng.choice([16, 16, 16, 8, 13, 32, 24, 64, 128, 256, 1, 2])
        G = rng.choice([1, 1, 2, 4])
        D = G * rng.choice([1, 3, 8, 16, 40, 48, 80, 81, 100, 160, 170] + ([240, 481] if big else []))
        H = P = 0
        if N <= 32 and rng.random() < 0.3:
            conv = rng.choice([1, 2, 3, 4])
        env["SSM_SCAN_MIXED"] = rng.choice(["", "0", "1", "48"])
    else:
        N = rng.choice([32, 64, 128] if mh_conv else [32, 64, 128, 16, 48, 256, 1])
        G = rng.choice([1, 2])
        H = G * rng.choice([1, 2, 3])
        P = rng.choice([16, 32, 48, 64, 128] if mh_conv else [16, 32, 48, 64, 8, 128, 3])
        D = H * P
        if rng.random() < 0.2 and not mh_conv:
            env["SSM_SCAN_SSD"] = "0"
        if rng.random() < 0.2:
            env["SSM_SSD_PS"] = "16"
        # the input stage runs where the chunked kernel does
        if io == "bf16" and N in (32, 64, 128) and P % 16 == 0 and "SSM_SCAN_SSD" not in env and \
                (mh_conv or rng.random() < 0.3):
            conv = rng.choice([1, 2, 3, 4])
    if rng.random() < 0.3:
        env["SSM_SCAN_SEGMENTS"] = str(rng.choice([1, 2, 3, 5, 9]))
    return dict(layout=layout, io=io, B=B, L=L, D=D, N=N, G=G, H=H, P=P, conv=conv, env=env,
                disc=rng.choice(["delta_b", "delta_b", "zoh"]),
                opts=dict(has_z=rng.random() < 0.7, has_D=rng.random() < 0.8, has_bias=rng.random() < 0.8,
                          has_h0=rng.random() < 0.6,
                          delta_kind=rng.choice(["small", "small", "wide", "long", "zero"])),
                softplus=rng.random() < 0.85, seed=rng.randrange(1 << 20), decode=rng.random() < 0.15,
                inplace=rng.random() < 0.5, conv_state=rng.random() < 0.5) if not mh_conv else \
        dict(layout=layout, io=io, B=B, L=L, D=D, N=N, G=G, H=H, P=P, conv=conv, env=env,
             disc=rng.choice(["delta_b", "delta_b", "zoh"]),
             opts=dict(has_z=rng.random() < 0.7, has_D=rng.random() < 0.8, has_bias=rng.random() < 0.8,
                       has_h0=rng.random() < 0.6, delta_kind=rng.choice(["small", "small", "wide", "long", "zero"])),
             softplus=rng.random() < 0.85, seed=rng.randrange(1 << 20), decode=False, inplace=False,
             conv_state=rng.random() < 0.5)


def run_case(k, monkeypatch):
    for key in ENV_KEYS:
        monkeypatch.delenv(key, raising=False)
    for key, v in k["env"].items():
        if v:
            monkeypatch.setenv(key, v)
    layout, io = k["layout"], k["io"]
    decode = k["decode"]
    opts = dict(k["opts"], has_h0=True) if decode else k["opts"]
    c = make_case("random", layout=layout, io_dtype=io, batch=k["B"], seqlen=1 if decode else k["L"], dim=k["D"],
                  dstate=k["N"], nheads=k["H"], headdim=k["P"], ngroups=k["G"], seed=k["seed"],
                  A_kind="head_uniform" if layout == "blhp" else "lognormal", **opts)
    c.softplus = k["softplus"]
    if not c.softplus:   # the step is delta itself: positive and small
        c.tensors["delta"] = (c.tensors["delta"].float().abs() * 0.05).to(c.tensors["delta"].dtype)
        c.tensors["delta_bias"] = None
    dev = torch.device("cuda:0")
    T = {key: (None if v is None else v.to(dev)) for key, v in c.tensors.items()}
    f = lambda key: None if c.tensors[key] is None else c.tensors[key].numpy()
    kw = dict(layout=layout, io_dtype=io, ngroups=k["G"], discretization="zoh" if k["disc"] == "zoh" else "euler")
    cs = cs_ref = None
    if decode:   # one step on the carried state h0: the step's inputs are the sequence's only step
        first = (lambda t: None if t is None else t[:, :, 0].contiguous()) if layout == "bdl" else \
                (lambda t: None if t is None else t[:, 0].contiguous())
        bc = (lambda t: t[..., 0].contiguous()) if layout == "bdl" else (lambda t: t[:, 0].contiguous())
        h_in = T["h0"].clone()
        yq, h = scan.ssm_state_update(first(T["u"]), first(T["delta"]), T["A"], bc(T["B"]), bc(T["C"]), T["D"],
                                      first(T["z"]), T["delta_bias"], c.softplus, h_in, layout=layout,
                                      inplace=k["inplace"], discretization=k["disc"])
        y = yq.unsqueeze(2) if layout == "bdl" else yq.unsqueeze(1)
    elif k["conv"]:
        K = k["conv"]
        g = torch.Generator().manual_seed(k["seed"])
        cw = (torch.randn(k["D"], K, generator=g) * 0.5).contiguous()
        cb = (torch.randn(k["D"], generator=g) * 0.2).contiguous()
        csi = torch.randn(k["B"], k["D"], K - 1, generator=g).contiguous() if K > 1 and k["conv_state"] else None
        y, h, cs = scan.ssm_conv_scan_fwd(T["u"], cw.to(dev), cb.to(dev), T["delta"], T["A"], T["B"], T["C"], T["D"],
                                          T["z"], T["delta_bias"], c.softplus, T["h0"], discretization=k["disc"],
                                          conv_state_in=None if csi is None else csi.to(dev), want_conv_state=True,
                                          layout=layout)
        kw.update(conv_w=cw.numpy(), conv_b=cb.numpy(), conv_state_in=None if csi is None else csi.numpy(),
                  want_conv_state=True)
    else:
        y, h = scan.ssm_scan_fwd(T["u"], T["delta"], T["A"], T["B"], T["C"], T["D"], T["z"], T["delta_bias"],
                                 c.softplus, T["h0"], layout=layout, discretization=k["disc"])
    torch.cuda.synchronize()
    res = oracle.scan_f64(np_io(c.tensors["u"], io), np_io(c.tensors["delta"], io), f("A"),
                          np_io(c.tensors["B"], io), np_io(c.tensors["C"], io), f("D"), np_io(c.tensors["z"], io),
                          f("delta_bias"), c.softplus, f("h0"), **kw)
    yr, hr = res[:2]
    if cs is not None:   # the input stage's final state is a copy of raw inputs: exact
        assert np.array_equal(cs.double().cpu().numpy(), np.asarray(res[2], dtype=np.float64).reshape(tuple(cs.shape)))
    return scaled_err(y, yr), scaled_err(h, hr)


@pytest.mark.parametrize("seed,count,big,mh_conv", [(7, 150, False, False), (23, 60, True, False),
                                                   (41, 150, False, False), (59, 60, False, True)])
def test_random_cases(seed, count, big, mh_conv, monkeypatch):
    rng = random.Random(seed)
    bad = []
    for i in range(count):
        k = draw(rng, big, mh_conv)
        print(f"[gpu] random case {seed}/{i}: {k}", flush=True)
        ey, eh = run_case(k, monkeypatch)
        tol = TOL[k["io"]]
        if not (ey <= tol and eh <= tol):
            bad.append((i, ey, eh, k))
    assert not bad, f"{len(bad)} of {count} cases over the bound: {bad[:3]}"
