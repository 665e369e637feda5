#!/usr/bin/env python3
"""Benchmark of the selective-scan (S6) forward on one MI355X.

One step = one ssm_scan_fwd call over the whole workload batch (all of the
path: step size, discretisation, recurrence, readout, skip, gate, final
state), inputs already resident in HBM.  Three input sets are rotated so the
256 MB Infinity Cache cannot serve a repeated working set.

Prints ONE JSON line: metric/value (elements B*L*D*N per second), the
roofline of the scan kernel (measured live with HIP events on the launch
stream), and the fp64 CPU oracle timed on a bounded sample on host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan elements/s (B·L·D·N) + achieved HBM GB/s vs MI355X peak"
DEFAULT_WORKLOAD = "mamba2p8b_layer"

# MI355X figures used for the rooflines: vendor peaks; 32 fp32 lanes per SIMD per clock as
# measured for v_fmac_f32 on gfx950, transcendentals at a quarter of that.
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
CUS, SIMDS, LANES_PER_CLK, CLOCK_HZ = 256, 4, 32, 2.4e9
VALU_SLOT_PEAK = CUS * SIMDS * LANES_PER_CLK * CLOCK_HZ       # 78.64e12 fp32 lane-ops/s (= 157.3 TFLOP/s FMA)
TRANS_SLOTS = 4                                               # exp2/log2/rcp issue at 1/4 of the fp32 rate

# Algorithmic work of the path, in fp32 VALU slots.
#  per (b,d,t,n): exp(dt*A) [1 mul + 1 transcendental], dt*u*B [1 mul], h update [1 fma], readout [1 fma]
#  per (b,d,t)  : softplus [bias add, 1+e add, exp, log], dt*u [mul], D*u [fma],
#                 SiLU gate [exp, 1+e add, rcp, z*s mul, y*s mul]
#  multi-head layout: exp(dt*A) is per (b,t,h), so per element only dt*u*B, h update, readout.
#  exact zero-order hold (--discretization zoh): per (b,d,t,n) in the per-channel layout, x = dt*A [mul],
#                 expm1 from the exp [add], divide by x [rcp + mul], scale B̄ [mul]; per (b,t,h) in the
#                 multi-head layout (the factor is per head).
ZOH_SLOTS = 4 + TRANS_SLOTS
#  fused input stage (--conv K): per (b,d,t) K fma for the causal conv, SiLU [exp, 1+e add, rcp, mul].
def conv_slots(K):
    return K + 2 + 2 * TRANS_SLOTS if K else 0


def algorithmic_slots(case, zoh=False, conv_k=0) -> float:
    Bsz, L, Dm, N = case.batch, case.seqlen, case.dim, case.dstate
    has_z = case.tensors["z"] is not None
    per_row_step = (2 + 2 * TRANS_SLOTS) + 2 + ((3 + 2 * TRANS_SLOTS) if has_z else 0) + conv_slots(conv_k)
    if case.layout == "bdl":
        per_elem = 4 + TRANS_SLOTS + (ZOH_SLOTS if zoh else 0)
        return Bsz * L * Dm * (N * per_elem + per_row_step)
    per_elem = 3
    per_head_step = (2 + 2 * TRANS_SLOTS) + (1 + TRANS_SLOTS) + (ZOH_SLOTS if zoh else 0)
    per_chan_step = 2 + ((3 + 2 * TRANS_SLOTS) if has_z else 0)
    return Bsz * L * (Dm * (N * per_elem + per_chan_step) + case.nheads * per_head_step)


def ssd_form_flops(case, chunk: int = 64) -> float:
    """Matrix flops of the chunked (state-space-duality) form of the multi-head layout, counted
    once: per (b, h, chunk of Q steps) C B^T (Q x Q x N, the causal half), its decayed product
    with X (Q x Q x P, causal half), the carried state's readout C H (Q x N x P) and the chunk's
    state contribution B^T X (N x Q x P); FMA = 2 flops.  No operand splitting, no recomputation."""
    Bsz, L, H, P, N = case.batch, case.seqlen, case.nheads, case.headdim, case.dstate
    chunks = -(-L // chunk)
    Q = chunk
    macs = (Q * Q * N) / 2 + (Q * Q * P) / 2 + Q * N * P + N * Q * P
    return 2.0 * macs * Bsz * H * chunks


def algorithmic_bytes(case) -> int:
    """Each input read once, each output written once; B/C once per (b, t)."""
    T = case.tensors
    total = 0
    for k in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias", "h0"):
        if T[k] is not None:
            total += T[k].numel() * T[k].element_size()
    total += T["u"].numel() * T["u"].element_size()                  # y
    total += case.batch * case.dim * case.dstate * 4                 # h_last
    return total


def kernel_source_hash(workload: str) -> str:
    """Hash of the sources the workload's kernels are built from (the host API plus the
    kernel file of its path), so counters taken for one path stay valid while another changes."""
    from selective_state_space_02_amd.inputs import DECODE_CONFIGS
    if workload in DECODE_CONFIGS:
        kern = "update_kernels.hip"
    elif workload == "mamba2_multihead":
        kern = "ssd_kernels.hip"
    else:
        kern = "scan_kernels.hip"
    h = hashlib.sha256()
    for f in ("scan_api.cpp", "scan_plan.h", kern):
        src = open(os.path.join(ROOT, "selective_state_space_02_amd", "csrc", f), encoding="utf-8").read()
        # the code only: comments and blank space do not change a kernel
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, variant: str = ""):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they match this kernel.
    variant: "" or the path's options ("_zoh", "_conv4", "_zoh_conv4")."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}{variant}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(case, budget_s: float = 12.0, zoh: bool = False, conv=None):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload: the first
    batch items (whole) or, if one item is already over budget, the first channels of
    item 0, always over the full sequence.  Returns the dict for the JSON line."""
    import numpy as np
    import torch

    import oracle

    T = case.tensors
    io = case.io_dtype

    def np_io(t):
        if t is None:
            return None
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if io == "bf16" else t.numpy()

    def run(nb, nch, threads=None):
        """nb batch items; nch channels (BDL) or nch // headdim heads (BLHP)."""
        f = lambda t: None if t is None else t.contiguous().numpy()
        if case.layout == "bdl":
            x = lambda t: None if t is None else t[:nb, :nch]
            args = (np_io(x(T["u"])), np_io(x(T["delta"])), f(T["A"][:nch]), np_io(T["B"][:nb]), np_io(T["C"][:nb]),
                    f(None if T["D"] is None else T["D"][:nch]), np_io(x(T["z"])),
                    f(None if T["delta_bias"] is None else T["delta_bias"][:nch]), case.softplus,
                    f(None if T["h0"] is None else T["h0"][:nb, :nch]))
            elems = nb * case.seqlen * nch * case.dstate
        else:
            nh = max(1, nch // case.headdim)
            x = lambda t: None if t is None else t[:nb, :, :nh]
            nc = nh * case.headdim
            args = (np_io(x(T["u"])), np_io(x(T["delta"])), f(T["A"][:nh]), np_io(T["B"][:nb]), np_io(T["C"][:nb]),
                    f(None if T["D"] is None else T["D"][:nc]), np_io(x(T["z"])),
                    f(None if T["delta_bias"] is None else T["delta_bias"][:nh]), case.softplus,
                    f(None if T["h0"] is None else T["h0"][:nb, :nc]))
            elems = nb * case.seqlen * nc * case.dstate
        threads = threads or oracle.default_threads()
        t0 = time.perf_counter()
        extra = {}
        if conv is not None:                              # the fused input stage, same channels
            extra = dict(conv_w=conv[0][:nch], conv_b=conv[1][:nch])
        oracle.scan_f64(*args, nthreads=threads, layout=case.layout, io_dtype=io, ngroups=case.ngroups,
                        discretization="zoh" if zoh else "euler", **extra)
        return time.perf_counter() - t0, elems, threads

    probe_ch = 64 if case.layout == "bdl" else case.headdim
    dt, el, _ = run(1, probe_ch)
    rate = el / max(dt, 1e-6)
    per_item = case.seqlen * case.dim * case.dstate
    nb = int(min(case.batch, max(1, rate * budget_s // per_item)))
    if rate * budget_s >= per_item:
        nch, what = case.dim, f"batch items 0..{nb - 1} of {case.batch} (all channels)"
    else:
        nch = int(max(probe_ch, rate * budget_s / (case.seqlen * case.dstate)))
        if case.layout == "blhp":
            nch = max(case.headdim, (nch // case.headdim) * case.headdim)
        nch = min(nch, case.dim)
        what = f"batch item 0, first {nch} of {case.dim} channels"
    dt, el, threads = run(nb, nch)
    # one thread on about 1/threads of that sample (the first channels of item 0)
    nch1 = max(probe_ch, (nch * nb) // max(1, threads))
    if case.layout == "blhp":
        nch1 = max(case.headdim, (nch1 // case.headdim) * case.headdim)
    dt1, el1, _ = run(1, min(nch1, case.dim), threads=1)
    return {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, all {case.seqlen} steps, {case.dstate} states: {el:.3e} elements in {dt:.2f} s",
            "value_1thread": el1 / dt1,
            "sample_1thread": f"batch item 0, first {min(nch1, case.dim)} channels, 1 thread: {el1:.3e} elements in "
                              f"{dt1:.2f} s"}


def decode_bytes(case) -> int:
    """State read and written once, every other input read once, y written once."""
    T = case.tensors
    total = 2 * case.batch * case.dim * case.dstate * 4
    for k in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias"):
        if T[k] is not None:
            total += T[k].numel() * T[k].element_size()
    return total + T["u"].numel() * T["u"].element_size()


def decode_step_tensors(case, dev):
    """The workload's single time step in the state-update layouts."""
    T = {k: (None if v is None else v.to(dev)) for k, v in case.tensors.items()}
    if case.layout == "bdl":
        pick = lambda x: None if x is None else x[:, :, 0].contiguous()
        B, C = T["B"][..., 0].contiguous(), T["C"][..., 0].contiguous()
    else:
        pick = lambda x: None if x is None else x[:, 0].contiguous()
        B, C = pick(T["B"]), pick(T["C"])
    return dict(x=pick(T["u"]), delta=pick(T["delta"]), B=B, C=C, z=pick(T["z"]), A=T["A"], D=T["D"],
                bias=T["delta_bias"], h=T["h0"])


def cpu_baseline_decode(case, budget_s: float = 12.0):
    """The fp64 oracle's one-step scan, repeated on the whole batch within the budget."""
    import numpy as np
    import torch

    import oracle

    T = case.tensors
    io = case.io_dtype

    def np_io(t):
        if t is None:
            return None
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if io == "bf16" else t.numpy()

    f = lambda t: None if t is None else t.contiguous().numpy()
    args = (np_io(T["u"]), np_io(T["delta"]), f(T["A"]), np_io(T["B"]), np_io(T["C"]), f(T["D"]), np_io(T["z"]),
            f(T["delta_bias"]), case.softplus, f(T["h0"]))
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.scan_f64(*args, nthreads=threads, layout=case.layout, io_dtype=io, ngroups=case.ngroups)
        reps += 1
        dt = time.perf_counter() - t0
        if dt > budget_s or reps >= 200:
            break
    el = reps * case.elements
    return {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full one-step updates of the whole batch ({case.elements:.3e} elements each) "
                      f"in {dt:.2f} s"}


def bench_decode(args, case, dev):
    """Single-token state update: one step = one ssm_state_update call over the whole batch."""
    import torch

    from selective_state_space_02_amd import scan

    sets = []
    for i in range(max(1, args.rotate) * 4):     # states of 4x the rotation count: > 256 MB in total
        s = decode_step_tensors(case, dev)
        s["h"] = s["h"].clone()
        s["y"] = torch.empty_like(s["x"])
        sets.append(s)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % len(sets)]
        scan.ssm_state_update(s["x"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["bias"], case.softplus,
                              s["h"], layout=case.layout, inplace=True, y=s["y"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    launch_ms = sum(per_launch) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    abytes = decode_bytes(case)
    achieved = abytes / (launch_ms * 1e-3) / 1e9
    line = {
        "metric": "selective state update (decode) elements/s (B·D·N) + achieved HBM GB/s vs MI355X peak",
        "value": case.batch * case.dim * case.dstate / (ms_per_step * 1e-3),
        "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "layout": case.layout, "io_dtype": case.io_dtype,
                   "batch": case.batch, "dim": case.dim, "dstate": case.dstate, "nheads": case.nheads,
                   "headdim": case.headdim, "ngroups": case.ngroups},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(args.workload),
                     "kernel_ms": launch_ms, "kernel_ms_median": per_launch[len(per_launch) // 2],
                     "kernel_ms_min": per_launch[0], "algorithmic_bytes_per_launch": abytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(case, args.cpu_budget)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=3, help="input sets rotated through (defeats the 256 MB MALL)")
    ap.add_argument("--discretization", choices=("delta_b", "zoh"), default="delta_b",
                    help="B̄ = Δ·B (the workloads' definition) or the exact zero-order hold")
    ap.add_argument("--conv", type=int, default=0, metavar="K",
                    help="fuse a causal depthwise conv1d of width K (1..4) + SiLU in front of the scan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run only a plain copy of this many MiB (counter calibration), then exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the scan shards over "
              "batch x channel with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_02_amd import scan
    from selective_state_space_02_amd.inputs import DECODE_CONFIGS, make_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}))
        return

    case = make_config(args.workload)
    if args.workload in DECODE_CONFIGS:
        return bench_decode(args, case, dev)
    sets = []
    for i in range(max(1, args.rotate)):
        T = {k: (None if v is None else v.to(dev)) for k, v in case.tensors.items()}
        y = torch.empty_like(T["u"])
        h = torch.empty((case.batch, case.dim, case.dstate), dtype=torch.float32, device=dev)
        sets.append((T, y, h))
    dims = scan.make_dims(case.layout, case.io_dtype, case.batch, case.seqlen, case.dim, case.dstate,
                          case.nheads, case.headdim, case.ngroups, args.discretization)
    ws_bytes = scan.workspace_size(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    plan = scan.describe(dims)
    stream = torch.cuda.current_stream(dev)

    conv = None
    if args.conv:
        gen = torch.Generator().manual_seed(20260999)
        conv = ((torch.randn(case.dim, args.conv, generator=gen) * 0.5).to(dev),
                (torch.randn(case.dim, generator=gen) * 0.2).to(dev))

    def step(i):
        T, y, h = sets[i % len(sets)]
        if conv is not None:
            scan.ssm_conv_scan_fwd(T["u"], conv[0], conv[1], T["delta"], T["A"], T["B"], T["C"], T["D"], T["z"],
                                   T["delta_bias"], case.softplus, T["h0"], discretization=args.discretization,
                                   stream=stream)
            return
        scan.ssm_scan_fwd(T["u"], T["delta"], T["A"], T["B"], T["C"], T["D"], T["z"], T["delta_bias"],
                          case.softplus, T["h0"], layout=case.layout, y=y, h_last=h, workspace=ws, stream=stream,
                          discretization=args.discretization)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, synchronised on both sides; per-launch HIP events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    launch_ms = sum(per_launch) / args.steps

    ms_per_step = wall * 1e3 / args.steps
    elements = case.elements
    value = elements / (ms_per_step * 1e-3)

    slots = algorithmic_slots(case, zoh=args.discretization == "zoh", conv_k=args.conv)
    achieved = slots / (launch_ms * 1e-3) / 1e12
    peak = VALU_SLOT_PEAK / 1e12
    abytes = algorithmic_bytes(case) + (case.dim * (args.conv + 1) * 4 if args.conv else 0)
    variant = ("_zoh" if args.discretization == "zoh" else "") + (f"_conv{args.conv}" if args.conv else "")
    traffic = load_traffic(args.workload, variant)
    hbm_gbs = abytes / (launch_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "layout": case.layout, "io_dtype": case.io_dtype, "batch": case.batch,
                   "seqlen": case.seqlen, "dim": case.dim, "dstate": case.dstate, "nheads": case.nheads,
                   "headdim": case.headdim, "ngroups": case.ngroups, "discretization": args.discretization,
                   "conv_width": args.conv, "plan": plan},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel_ms": launch_ms, "kernel_ms_median": per_launch[len(per_launch) // 2],
                     "kernel_ms_min": per_launch[0], "algorithmic_ops_per_launch": slots,
                     "op": "fp32 VALU lane-issue slot (transcendental = 4)"},
        "hbm": {"algorithmic_bytes_per_launch": abytes, "achieved_GBs": hbm_gbs, "peak_GBs": HBM_PEAK_GBS,
                "frac": hbm_gbs / HBM_PEAK_GBS},
    }
    if "kernel=ssd" in plan:   # the chunked form runs its contractions on bf16 MFMA
        mf = ssd_form_flops(case) / (launch_ms * 1e-3) / 1e12
        line["mfma"] = {"achieved": mf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": mf / MFMA_BF16_PEAK_TFLOPS, "flops_per_launch": ssd_form_flops(case),
                        "op": "chunked-form matrix flops, each product counted once (dense bf16 peak)"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget, zoh=args.discretization == "zoh",
                                            conv=None if conv is None else (conv[0].cpu().numpy(),
                                                                            conv[1].cpu().numpy()))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
