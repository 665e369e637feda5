"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and shapes tensors; it holds none of the
scan's arithmetic, so both the HIP path and the fp64 oracle may use it.
Everything is generated with a seeded torch.Generator, on the CPU unless a case
asks for another device (cases too large to draw on the host), drawn in float32
and rounded to bfloat16 (round-to-nearest-even) where the case says so.
The step sizes come from the inverse of log(1+e^r); that inverse is the only
formula here and it only places the drawn values inside the wanted range.

Layouts (all contiguous):
  "bdl"  : u, delta, z: (B, D, L); B, C: (B, G, N, L); A: (D, N); delta_bias, D: (D,)
  "blhp" : u, z: (B, L, H, P); delta: (B, L, H); B, C: (B, L, G, N); A: (H,);
           delta_bias: (H,); D: (H*P,)
  h0: (B, D, N) float32 in both.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

SEED_BASE = 20260000

# Bias range and raw-step range that place softplus(raw + bias) inside [1e-3, 1e-1]:
# inverse softplus of 1e-3 is -6.9073 and of 1e-1 is -2.2522, raw is kept in [-2, 2].
_BIAS_LO, _BIAS_HI = -4.9073, -4.2522
_RAW_CLIP = 2.0


@dataclass
class Case:
    name: str
    layout: str                 # "bdl" or "blhp"
    io_dtype: str               # "f32" or "bf16"
    batch: int
    seqlen: int
    dim: int
    dstate: int
    nheads: int = 0
    headdim: int = 0
    ngroups: int = 1
    softplus: bool = True
    tensors: Dict[str, Optional[torch.Tensor]] = field(default_factory=dict)

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, std=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=g.device) * std


def _uniform(shape, g, lo, hi):
    return torch.rand(*shape, generator=g, dtype=torch.float32, device=g.device) * (hi - lo) + lo


_RESAMPLE_CHUNK = 1 << 28   # masked assignment is done per chunk (torch's fails past 2^31 elements)


def _truncated_normal(shape, g, clip):
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=g.device)
    flat = x.view(-1)
    for s in range(0, flat.numel(), _RESAMPLE_CHUNK):
        part = flat[s:s + _RESAMPLE_CHUNK]
        bad = part.abs() > clip
        while bool(bad.any()):
            part[bad] = torch.randn(int(bad.sum()), generator=g, dtype=torch.float32, device=g.device)
            bad = part.abs() > clip
    return x


def _inv_softplus(target: torch.Tensor) -> torch.Tensor:
    t = target.double()
    return torch.log(torch.expm1(t)).float()


def _io(x: torch.Tensor, io_dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if io_dtype == "bf16" else x.float()


def make_case(name="custom", *, layout="bdl", io_dtype="bf16", batch=1, seqlen=256, dim=64, dstate=16,
              nheads=0, headdim=0, ngroups=1, seed=1, has_z=True, has_D=True, has_bias=True,
              softplus=True, has_h0=False, A_kind="arange", delta_kind="small", device="cpu") -> Case:
    """General seeded case (tensors on `device`; the draws depend on the device's generator).

    A_kind: "arange" -> A[d, n] = -(n+1); "lognormal" -> -exp(N(0, 0.5));
            "head_uniform" -> per head -exp(U(0, 2.7)).
    delta_kind: "small" -> raw ~ N(0,1) clipped to [-2,2] with bias ~ U(-4.907, -4.252)
                           (softplus gives [1e-3, 1e-1]); "long" -> 10% of positions with a
                           step near 1e-4 and the rest in [1e-2, 1e-1] (no bias);
                           "zero" -> raw = 0; "wide" -> raw ~ N(0, 3), bias 0.
    """
    g = _gen(seed, device)
    c = Case(name, layout, io_dtype, batch, seqlen, dim, dstate, nheads, headdim, ngroups, softplus)
    T = {}
    N = dstate
    if layout == "bdl":
        xs = (batch, dim, seqlen)
        bcs = (batch, ngroups, N, seqlen)
        dts = xs
        nbias = dim
    else:
        assert nheads * headdim == dim
        xs = (batch, seqlen, nheads, headdim)
        bcs = (batch, seqlen, ngroups, N)
        dts = (batch, seqlen, nheads)
        nbias = nheads
    T["u"] = _io(_normal(xs, g), io_dtype)
    # step sizes
    if delta_kind == "small":
        raw = _truncated_normal(dts, g, _RAW_CLIP)
        bias = _uniform((nbias,), g, _BIAS_LO, _BIAS_HI) if has_bias else None
        if bias is None:
            raw = raw + (_BIAS_LO + _BIAS_HI) / 2
    elif delta_kind == "long":
        mask = torch.rand(*dts, generator=g, device=g.device) < 0.1
        lo_s, hi_s = math.log(5e-5), math.log(2e-4)
        lo_l, hi_l = math.log(1e-2), math.log(1e-1)
        tgt = torch.where(mask, torch.exp(_uniform(dts, g, lo_s, hi_s)), torch.exp(_uniform(dts, g, lo_l, hi_l)))
        raw = _inv_softplus(tgt)
        bias = None
    elif delta_kind == "zero":
        raw = torch.zeros(dts, device=g.device)
        bias = torch.zeros(nbias, device=g.device) if has_bias else None
    elif delta_kind == "wide":
        raw = _normal(dts, g, 3.0)
        bias = torch.zeros(nbias, device=g.device) if has_bias else None
    else:
        raise ValueError(delta_kind)
    T["delta"] = _io(raw, io_dtype)
    T["delta_bias"] = bias.float() if bias is not None else None
    # A
    if layout == "bdl":
        if A_kind == "arange":
            A = -torch.arange(1, N + 1, dtype=torch.float32, device=g.device).repeat(dim, 1)
        elif A_kind == "lognormal":
            A = -torch.exp(_normal((dim, N), g, 0.5))
        else:
            raise ValueError(A_kind)
    else:
        A = -torch.exp(_uniform((nheads,), g, 0.0, 2.7))
    T["A"] = A.contiguous()
    T["B"] = _io(_normal(bcs, g), io_dtype)
    T["C"] = _io(_normal(bcs, g), io_dtype)
    if has_D:
        if layout == "bdl":
            T["D"] = _normal((dim,), g)
        else:
            T["D"] = _normal((nheads,), g).repeat_interleave(headdim).contiguous()
    else:
        T["D"] = None
    T["z"] = _io(_normal(xs, g), io_dtype) if has_z else None
    T["h0"] = _normal((batch, dim, N), g) if has_h0 else None
    c.tensors = T
    return c


# The five workloads, with their sizes.  Names describe what each one is.
CONFIGS = {
    "tiny_f32": dict(layout="bdl", io_dtype="f32", batch=1, seqlen=256, dim=64, dstate=16,
                     has_z=False, has_D=True, has_bias=True, A_kind="arange", delta_kind="small"),
    "mamba130m_layer": dict(layout="bdl", io_dtype="bf16", batch=8, seqlen=2048, dim=1536, dstate=16,
                            has_z=True, has_D=True, has_bias=True, A_kind="arange", delta_kind="small"),
    "mamba2p8b_layer": dict(layout="bdl", io_dtype="bf16", batch=4, seqlen=2048, dim=5120, dstate=16,
                            has_z=True, has_D=True, has_bias=True, A_kind="lognormal", delta_kind="small"),
    "long_carry": dict(layout="bdl", io_dtype="bf16", batch=1, seqlen=131072, dim=2560, dstate=16,
                       has_z=False, has_D=True, has_bias=False, has_h0=True, A_kind="lognormal",
                       delta_kind="long"),
    "mamba2_multihead": dict(layout="blhp", io_dtype="bf16", batch=2, seqlen=8192, dim=5120, dstate=128,
                             nheads=80, headdim=64, ngroups=1, has_z=True, has_D=True, has_bias=True,
                             A_kind="head_uniform", delta_kind="small"),
}
CONFIG_IDS = {name: i + 1 for i, name in enumerate(CONFIGS)}

# Single-token decode (state update) workloads: one step for a serving batch of
# sequences, with the channel/state shapes of the Mamba-2.8B-shaped layer and of
# the multi-head layer.  The state is read and written once per step.
DECODE_CONFIGS = {
    "mamba2p8b_decode": dict(layout="bdl", io_dtype="bf16", batch=64, seqlen=1, dim=5120, dstate=16,
                             has_z=True, has_D=True, has_bias=True, has_h0=True, A_kind="lognormal",
                             delta_kind="small"),
    "mamba2_decode": dict(layout="blhp", io_dtype="bf16", batch=16, seqlen=1, dim=5120, dstate=128,
                          nheads=80, headdim=64, ngroups=1, has_z=True, has_D=True, has_bias=True, has_h0=True,
                          A_kind="head_uniform", delta_kind="small"),
}
DECODE_IDS = {name: 101 + i for i, name in enumerate(DECODE_CONFIGS)}


def make_config(name: str, seed: Optional[int] = None) -> Case:
    if name in DECODE_CONFIGS:
        kw = dict(DECODE_CONFIGS[name])
        base_id = DECODE_IDS[name]
    else:
        kw = dict(CONFIGS[name])
        base_id = CONFIG_IDS[name]
    if seed is None:
        seed = SEED_BASE + base_id
    return make_case(name, seed=seed, **kw)
