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

# MI355X figures used for the rooflines.  Vendor peaks for HBM and the bf16 matrix units.
# The fp32 vector peak is derived from the unit counts and the boost clock: 256 CUs x 4 SIMDs
# x 16 fp32 lanes per clock x 2.4 GHz = 39.3 T lane-ops/s (78.6 TFLOP/s with FMA = 2; the
# published 157.3 TFLOP/s needs packed fp32, which this library does not emit).  A
# transcendental (v_exp_f32, v_log_f32, v_rcp_f32) retires 8 lanes per clock, i.e. it holds
# the VALU for two fp32 issue slots, and does not overlap with fp32 work.  Both rates are
# measured by `bench.py --valu-rates` (profiles/valu_rates_gfx950.txt).
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
CUS, SIMDS, CLOCK_HZ = 256, 4, 2.4e9
FP32_LANES_PER_CLK, TRANS_LANES_PER_CLK = 16, 8
VALU_SLOT_PEAK = CUS * SIMDS * FP32_LANES_PER_CLK * CLOCK_HZ   # 39.32e12 fp32 lane-ops/s
TRANS_PEAK = CUS * SIMDS * TRANS_LANES_PER_CLK * CLOCK_HZ      # 19.66e12 transcendentals/s
TRANS_SLOTS = FP32_LANES_PER_CLK // TRANS_LANES_PER_CLK        # VALU slots one transcendental holds

# Algorithmic work of the path.  "ops" are fp32 VALU instructions per lane, "trans" the
# transcendentals among them (each counted as TRANS_SLOTS slots in the ALU bound).
#  per (b,d,t,n): dt*A [mul], exp2 [trans], (dt*u)*B [mul], h update [fma], readout [fma]
#  per (b,d,t)  : dt = softplus(delta + bias) [add, mul, exp2, add, log2, max, fma],
#                 dt*u [mul], D*u [fma], SiLU gate [mul, exp2, add, rcp, mul, mul]
#  multi-head layout: exp(dt*A) is per (b,t,h), so per element only dt*u*B, h update, readout.
#  exact zero-order hold: per element x = dt*A [mul], expm1 = a - 1 [add], 1/x [rcp],
#                 (a-1)/x [mul], scale the input [mul]; per (b,t,h) in the multi-head layout.
#  fused input stage of width K: per (b,d,t) K fma for the causal conv, SiLU [mul, exp2, add, rcp, mul].
ELEM_OPS, ELEM_TRANS = 5, 1
SOFTPLUS_OPS, SOFTPLUS_TRANS = 7, 2
GATE_OPS, GATE_TRANS = 6, 2
ZOH_OPS, ZOH_TRANS = 5, 1


def conv_ops(K):
    return (K + 5, 2) if K else (0, 0)


def algorithmic_ops(case, zoh=False, conv_k=0):
    """(fp32 VALU ops, transcendentals) per call of the scan as the method defines it."""
    Bsz, L, Dm, N = case.batch, case.seqlen, case.dim, case.dstate
    has_z = case.tensors["z"] is not None
    sp = (SOFTPLUS_OPS, SOFTPLUS_TRANS) if case.softplus else (1, 0)          # the bias add alone without softplus
    gate = (GATE_OPS, GATE_TRANS) if has_z else (0, 0)
    cv = conv_ops(conv_k)
    row_ops = sp[0] + 1 + 1 + gate[0] + cv[0]            # + dt*u, D*u
    row_trans = sp[1] + gate[1] + cv[1]
    if case.layout == "bdl":
        el_ops = ELEM_OPS + (ZOH_OPS if zoh else 0)
        el_trans = ELEM_TRANS + (ZOH_TRANS if zoh else 0)
        rows = Bsz * L * Dm
        return rows * (N * el_ops + row_ops), rows * (N * el_trans + row_trans)
    # multi-head: decay per (b,t,h); softplus per (b,t,h); dt*u, D*u, gate per (b,t,d)
    head_ops = sp[0] + 2 + (ZOH_OPS if zoh else 0)       # + dt*A mul, exp2
    head_trans = sp[1] + 1 + (ZOH_TRANS if zoh else 0)
    chan_ops = 2 + gate[0]
    ops = Bsz * L * (Dm * (N * 3 + chan_ops) + case.nheads * head_ops)
    trans = Bsz * L * (Dm * gate[1] + case.nheads * head_trans)
    return ops, trans


def valu_slots(ops, trans):
    """fp32 VALU issue slots: every op one slot, a transcendental TRANS_SLOTS."""
    return ops + (TRANS_SLOTS - 1) * trans


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


def host_cpus():
    """The host's CPU counts beside the threads the oracle ran on: the oracle uses every core
    this process may run on, up to 16 (the host CPU share of one GPU on an 8-GPU MI355X node)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"host_cpu_count": os.cpu_count(), "usable_cpus": usable, "cpu_share_per_gpu": 16}


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
    return {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle", **host_cpus(),
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
    return {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle", **host_cpus(),
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


def valu_rates():
    """Issue rates behind the ALU and transcendental bounds: each kind of instruction alone on
    8 independent chains per lane, at 1 to 8 waves per SIMD, plus the scan's own element mix
    and 4 fma + 1 exp (to show that a transcendental and fp32 work add up); HBM read and copy."""
    import ctypes

    from selective_state_space_02_amd import build as hipbuild

    if not os.path.exists(hipbuild.RATES_LIB):
        raise RuntimeError(f"{hipbuild.RATES_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(hipbuild.RATES_LIB)
    lib.ssm_rates_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.ssm_rates_hbm.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    kinds = {0: "v_fma_f32", 1: "v_mul_f32", 2: "v_exp_f32", 3: "v_log_f32", 4: "v_rcp_f32",
             5: "scan element (mul, exp2, mul, fma, fma)", 6: "4 fma + 1 exp2"}
    for k, name in kinds.items():
        for w in (1, 2, 4, 8):
            res = (ctypes.c_double * 4)()
            rc = lib.ssm_rates_run(k, w, res)
            if rc != 0:
                raise RuntimeError(f"ssm_rates_run({k}, {w}) failed: hipError {rc}")
            ms, ghz, per_s, cyc = list(res)
            print(json.dumps({"rate": name, "waves_per_simd": w, "ms": round(ms, 4), "clock_GHz": round(ghz, 3),
                              "units_per_s_per_simd": per_s, "cycles_per_unit_per_simd": round(cyc, 3),
                              "lanes_per_clk": round(64 / cyc, 2)}), flush=True)
    res = (ctypes.c_double * 2)()
    rc = lib.ssm_rates_hbm(1024, res)
    if rc != 0:
        raise RuntimeError(f"ssm_rates_hbm failed: hipError {rc}")
    print(json.dumps({"rate": "HBM 1 GiB", "read_GBs": round(res[0], 1), "copy_GBs": round(res[1], 1)}), flush=True)


# ---------------------------------------------------------------------------------------------
# rocprofv3 summaries (profiles/): text tables and the HBM-traffic record load_traffic reads.
# Input: one directory per workload holding the CSV output (-f csv) of
#   trace/          rocprofv3 --kernel-trace --stats -o trace -- python3 bench.py <args> --steps 20 --warmup 5 --no-cpu-baseline
#   pmc_FETCH_SIZE/ rocprofv3 --pmc FETCH_SIZE -o pmc -- python3 bench.py <args> --steps 3 --warmup 1 --rotate 1 --no-cpu-baseline
#   pmc_WRITE_SIZE/ the same with WRITE_SIZE
#   sq1/ sq2/ sq3/  (optional) the same with the SQ / GRBM counter sets of SQ_PASSES
# and a calibration directory with pmc_FETCH_SIZE/ and pmc_WRITE_SIZE/ of
#   rocprofv3 --pmc <C> -o pmc -- python3 bench.py --calib-copy-mb 512
SQ_PASSES = [
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_ACTIVE_INST_LDS "
    "SQ_WAIT_INST_LDS",
    "SQ_WAIT_INST_ANY SQ_INSTS_VALU_TRANS_F32 SQ_LDS_BANK_CONFLICT SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE GRBM_COUNT",
    "SQ_WAIT_ANY SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
    "SQ_INSTS_SMEM SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VMEM",
]


def _short_kernel(name: str) -> str:
    return name.replace("ssm::(anonymous namespace)::", "").replace("(ssm::KParams)", "")


def _csv_rows(path: str):
    import csv
    import glob
    hits = sorted(glob.glob(os.path.join(path, "**", "*.csv"), recursive=True))
    return [(f, list(csv.DictReader(open(f, newline="")))) for f in hits]


def _pmc_per_dispatch(path: str):
    """{kernel: {counter: mean value per dispatch}} from a --pmc run's counter_collection.csv."""
    acc = {}
    for f, rows in _csv_rows(path):
        if not f.endswith("counter_collection.csv"):
            continue
        for r in rows:
            k = r["Kernel_Name"]
            key = (r["Dispatch_Id"], r["Counter_Name"])
            d = acc.setdefault(k, {})
            d.setdefault(r["Counter_Name"], {})
            d[r["Counter_Name"]][key] = d[r["Counter_Name"]].get(key, 0.0) + float(r["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def profile_summary(args) -> None:
    """Write profiles/<prefix>_<tag>.txt, pmc_<tag>.json and (with SQ passes) sq_counters_<tag>.txt."""
    from selective_state_space_02_amd.inputs import DECODE_CONFIGS, make_config

    src, tag = args.profile_summary, args.profile_tag
    wl_args = f"--workload {args.workload}"
    if args.discretization != "delta_b":
        wl_args += f" --discretization {args.discretization}"
    if args.conv:
        wl_args += f" --conv {args.conv}"
    variant = ("_zoh" if args.discretization == "zoh" else "") + (f"_conv{args.conv}" if args.conv else "")
    decode = args.workload in DECODE_CONFIGS
    what = "state update" if decode else "selective scan"
    prefix = "update" if decode else "scan"
    bench_cmd = "python3 /root/repo/bench.py"
    cmds = [f"rocprofv3 --kernel-trace --stats -f csv -d <out>/trace -o trace -- {bench_cmd} {wl_args} --steps 20 "
            f"--warmup 5 --no-cpu-baseline"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"rocprofv3 --pmc {c} -f csv -d <out>/pmc_{c} -o pmc -- {bench_cmd} {wl_args} --steps 3 "
                    f"--warmup 1 --rotate 1 --no-cpu-baseline")
    cmds.append(f"rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE -f csv -d <calib>/pmc_<C> -o pmc -- {bench_cmd} "
                f"--calib-copy-mb 512")

    # kernel trace
    stats = []
    for f, rows in _csv_rows(os.path.join(src, "trace")):
        if f.endswith("kernel_stats.csv"):
            stats = rows
    lib = [r for r in stats if "ssm::" in r["Name"]]
    if not lib:
        raise SystemExit(f"no library kernels in the trace under {src}")
    avg_us = {_short_kernel(r["Name"]): float(r["AverageNs"]) / 1e3 for r in lib}
    dominant = max(lib, key=lambda r: float(r["TotalDurationNs"]))

    # HBM counters, calibrated by a plain copy of known size
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        per = _pmc_per_dispatch(os.path.join(args.profile_calib, f"pmc_{c}"))
        cal[c] = max(v.get(c, 0.0) for k, v in per.items() if "copyBuffer" in k)
    calib_kib = 512 * 1024
    fetch_factor, write_factor = calib_kib / cal["FETCH_SIZE"], calib_kib / cal["WRITE_SIZE"]
    cnt = {c: _pmc_per_dispatch(os.path.join(src, f"pmc_{c}")) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    case = make_config(args.workload)
    abytes = algorithmic_bytes(case) + (case.dim * (args.conv + 1) * 4 if args.conv else 0)

    w = 70
    out = [f"# rocprofv3 summary: {what}, workload {args.workload}{' (' + variant[1:] + ')' if variant else ''}",
           "# made on one MI355X (gfx950)",
           "# commands (run from /tmp with TMPDIR=/tmp, repo at /root/repo; text made by",
           f"#   python3 bench.py --profile-summary <out> --profile-calib <calib> --profile-tag {tag} {wl_args}):"]
    out += [f"#   {c}" for c in cmds]
    out += ["", "## kernel trace (--kernel-trace --stats), durations in microseconds",
            f"{'kernel':<{w}} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in stats:
        out.append(f"{_short_kernel(r['Name'])[:w]:<{w}} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                   f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.1f}")
    out += ["", "## HBM counters per dispatch (KiB as reported; calibrated by a plain 512 MiB copy)",
            f"copy kernel FETCH_SIZE {cal['FETCH_SIZE']:.0f} KiB for {calib_kib} KiB read  -> factor {fetch_factor:.3f}",
            f"copy kernel WRITE_SIZE {cal['WRITE_SIZE']:.0f} KiB for {calib_kib} KiB written -> factor {write_factor:.3f}"]
    total = 0.0
    for k in sorted(cnt["FETCH_SIZE"]):
        if "ssm::" not in k:
            continue
        fk = cnt["FETCH_SIZE"][k]["FETCH_SIZE"]
        wk = cnt["WRITE_SIZE"].get(k, {}).get("WRITE_SIZE", 0.0)
        fb, wb = fk * 1024 * fetch_factor, wk * 1024 * write_factor
        total += fb + wb
        out.append(f"{_short_kernel(k)[:w]:<{w}} FETCH {fk:>10.0f} KiB -> {fb / 1e6:>8.2f} MB   "
                   f"WRITE {wk:>10.0f} KiB -> {wb / 1e6:>8.2f} MB")
    out.append(f"HBM bytes per call (all library kernels of one call): {total / 1e6:.2f} MB; algorithmic bytes "
               f"{abytes / 1e6:.2f} MB; ratio {total / abytes:.3f}")
    outdir = args.profile_out or os.path.join(ROOT, "profiles")
    os.makedirs(outdir, exist_ok=True)
    with open(os.path.join(outdir, f"{prefix}_{tag}.txt"), "w") as fh:
        fh.write("\n".join(out) + "\n")
    rec = {"workload": args.workload, "options": variant[1:], "kernel_source_hash": kernel_source_hash(args.workload),
           "hbm_bytes_per_launch": total, "algorithmic_bytes_per_launch": abytes, "fetch_factor": fetch_factor,
           "write_factor": write_factor, "kernel_avg_us": avg_us}
    with open(os.path.join(outdir, f"pmc_{args.workload}{variant}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")

    # SQ counters of the dominant kernel, if the three passes were taken
    if not all(os.path.isdir(os.path.join(src, f"sq{i}")) for i in (1, 2, 3)):
        return
    kname = dominant["Name"]
    sq = {}
    for i in (1, 2, 3):
        sq.update(_pmc_per_dispatch(os.path.join(src, f"sq{i}")).get(kname, {}))
    kus = float(dominant["AverageNs"]) / 1e3
    cyc = sq["GRBM_GUI_ACTIVE"] / 8.0            # per-XCD clock cycles of the dispatch
    simds, cus = CUS * SIMDS, CUS
    waves = sq["SQ_WAVES"]
    sq_cmds = [f"rocprofv3 --pmc {p} -f csv -d <out>/sq{i + 1} -o pmc -- {bench_cmd} {wl_args} --steps 3 --warmup 1 "
               f"--rotate 1 --no-cpu-baseline" for i, p in enumerate(SQ_PASSES)]
    lines = [f"# SQ / GRBM counters per dispatch of {_short_kernel(kname)}, workload {args.workload}{variant}",
             "# made on one MI355X (gfx950); counter units as rocprofv3 reports them",
             "# commands (from /tmp with TMPDIR=/tmp, repo at /root/repo), three passes:"]
    lines += [f"#   {c}" for c in sq_cmds]
    lines.append("")
    lines += [f"{k:<28} {v:>14.6g}" for k, v in sorted(sq.items())]
    mf = sq.get("SQ_INSTS_MFMA", 0.0)
    lines += ["", "derived (GRBM_GUI_ACTIVE sums the 8 XCDs; SQ_ACTIVE_*, SQ_WAIT_*, SQ_WAVE_CYCLES are in quad-cycles):",
              f"  shader clock over the dispatch   {cyc / (kus * 1e3):.2f} GHz  (GRBM_GUI_ACTIVE/8 over the {kus:.1f} us "
              f"average of the kernel trace)",
              f"  VALU instructions per wave       {sq['SQ_INSTS_VALU'] / waves:.0f}  "
              f"({100 * sq['SQ_INSTS_VALU_TRANS_F32'] / sq['SQ_INSTS_VALU']:.0f}% transcendental)",
              f"  VALU busy per SIMD               {100 * 4 * sq['SQ_ACTIVE_INST_VALU'] / (simds * cyc):.0f}%  "
              f"(4*SQ_ACTIVE_INST_VALU / ({simds} SIMDs x cycles))",
              f"  cycles per VALU instruction      {4 * sq['SQ_ACTIVE_INST_VALU'] / sq['SQ_INSTS_VALU']:.2f}  "
              f"(per wave, issue to completion)",
              f"  LDS instructions per wave        {sq['SQ_INSTS_LDS'] / waves:.0f};  LDS busy per CU "
              f"{100 * 4 * sq['SQ_ACTIVE_INST_LDS'] / (cus * cyc):.0f}% of wave-cycles summed over its 4 SIMDs",
              f"  LDS bank-conflict cycles         "
              f"{100 * sq['SQ_LDS_BANK_CONFLICT'] / max(1.0, 4 * sq['SQ_ACTIVE_INST_LDS']):.0f}% of LDS-active cycles",
              f"  wave time waiting to issue       {100 * sq['SQ_WAIT_INST_ANY'] / sq['SQ_WAVE_CYCLES']:.0f}% (any), "
              f"{100 * sq['SQ_WAIT_INST_LDS'] / sq['SQ_WAVE_CYCLES']:.0f}% (LDS)",
              f"  wave time waiting (s_waitcnt)    {100 * sq['SQ_WAIT_ANY'] / sq['SQ_WAVE_CYCLES']:.0f}%",
              f"  SALU instructions per wave       {sq['SQ_INSTS_SALU'] / waves:.0f}"]
    if mf:
        lines += [f"  MFMA instructions per wave       {mf / waves:.0f};  MFMA busy per SIMD "
                  f"{100 * sq['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * cyc):.0f}%",
                  f"    (SQ_VALU_MFMA_BUSY_CYCLES / ({simds} SIMDs x cycles); the counter sums the SIMDs: it equals",
                  f"     SQ_INSTS_MFMA x {sq['SQ_VALU_MFMA_BUSY_CYCLES'] / mf:.1f} cycles per 16x16x32 bf16 MFMA)"]
    with open(os.path.join(outdir, f"sq_counters_{tag}.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


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
    ap.add_argument("--valu-rates", action="store_true",
                    help="measure the fp32 / transcendental issue rates, clock and HBM stream rates the "
                         "rooflines rest on (libssm_rates.so), print one JSON line per measurement, then exit")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="summarise the rocprofv3 CSV output under DIR into profiles/ (no GPU), then exit")
    ap.add_argument("--profile-calib", metavar="DIR", help="calibration copy counters for --profile-summary")
    ap.add_argument("--profile-tag", help="name of the summary files (default: the workload)")
    ap.add_argument("--profile-out", metavar="DIR", help="where --profile-summary writes (default: profiles/)")
    args = ap.parse_args()

    if args.profile_summary:
        args.profile_tag = args.profile_tag or args.workload
        return profile_summary(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the scan shards over "
              "batch x channel with no communication); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_02_amd import scan
    from selective_state_space_02_amd.inputs import DECODE_CONFIGS, make_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.valu_rates:
        return valu_rates()

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
                                   layout=case.layout, stream=stream)
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

    ops, trans = algorithmic_ops(case, zoh=args.discretization == "zoh", conv_k=args.conv)
    slots = valu_slots(ops, trans)
    abytes = algorithmic_bytes(case) + (case.dim * (args.conv + 1) * 4 if args.conv else 0)
    variant = ("_zoh" if args.discretization == "zoh" else "") + (f"_conv{args.conv}" if args.conv else "")
    traffic = load_traffic(args.workload, variant)
    kernel_s = launch_ms * 1e-3
    hbm_gbs = abytes / kernel_s / 1e9
    hbm = {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_gbs / HBM_PEAK_GBS,
           "traffic": traffic, "algorithmic_bytes_per_launch": abytes}
    alu = {"bound": "alu", "achieved": slots / kernel_s / 1e12, "peak": VALU_SLOT_PEAK / 1e12, "unit": "TOP/s",
           "frac": slots / kernel_s / VALU_SLOT_PEAK, "algorithmic_ops_per_launch": slots,
           "op": f"fp32 VALU lane-issue slot (fma/mul/add = 1, transcendental = {TRANS_SLOTS}); peak = 256 CUs x 4 "
                 f"SIMDs x {FP32_LANES_PER_CLK} fp32 lanes/clk x 2.4 GHz"}
    trn = {"bound": "trans", "achieved": trans / kernel_s / 1e12, "peak": TRANS_PEAK / 1e12, "unit": "T/s",
           "frac": trans / kernel_s / TRANS_PEAK, "transcendentals_per_launch": trans,
           "op": f"v_exp_f32 / v_log_f32 / v_rcp_f32; peak = 256 CUs x 4 SIMDs x {TRANS_LANES_PER_CLK} lanes/clk x 2.4 GHz"}
    ssd = "kernel=ssd" in plan
    if ssd:
        # the chunked form regroups the recurrence onto bf16 MFMA: the scan-form VALU count is not
        # work this kernel issues, so the line reports HBM with the matrix units beside it
        flops = ssd_form_flops(case)
        mf = flops / kernel_s / 1e12
        roof = hbm
        extra = {"mfma": {"bound": "mfma", "achieved": mf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": mf / MFMA_BF16_PEAK_TFLOPS, "flops_per_launch": flops,
                          "op": "chunked-form matrix flops, each product counted once (dense bf16 peak)"}}
        dtype = "bf16"   # matrix operands (hi/lo split); accumulation and the elementwise work in fp32
    else:
        # one lane per (channel, state) in fp32: bound by VALU issue, with HBM and the
        # transcendental pipe beside it
        roof = alu
        extra = {"hbm": hbm, "trans": trn}
        dtype = "f32"
    roof = dict(roof)
    if roof["bound"] != "hbm":
        roof["traffic"] = traffic
    roof.update({"kernel_ms": launch_ms, "kernel_ms_median": per_launch[len(per_launch) // 2],
                 "kernel_ms_min": per_launch[0]})

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
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "layout": case.layout, "io_dtype": case.io_dtype, "batch": case.batch,
                   "seqlen": case.seqlen, "dim": case.dim, "dstate": case.dstate, "nheads": case.nheads,
                   "headdim": case.headdim, "ngroups": case.ngroups, "discretization": args.discretization,
                   "conv_width": args.conv, "plan": plan},
        "roofline": roof,
        **extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget, zoh=args.discretization == "zoh",
                                            conv=None if conv is None else (conv[0].cpu().numpy(),
                                                                            conv[1].cpu().numpy()))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
