"""The roofline arithmetic of bench.py (no GPU): the algorithmic op counts per call and the
peaks derived from the unit counts, for the workloads the bench line reports."""
from types import SimpleNamespace

import bench


def make_config(name):
    """Shapes and options of the workloads (the bench model reads nothing else)."""
    shapes = {"mamba2p8b_layer": dict(layout="bdl", batch=4, seqlen=2048, dim=5120, dstate=16, nheads=0, headdim=0, z=True),
              "long_carry": dict(layout="bdl", batch=1, seqlen=131072, dim=2560, dstate=16, nheads=0, headdim=0, z=False),
              "mamba2_multihead": dict(layout="blhp", batch=2, seqlen=8192, dim=5120, dstate=128, nheads=80, headdim=64,
                                       z=True)}[name]
    z = shapes.pop("z")
    return SimpleNamespace(softplus=True, tensors={"z": object() if z else None}, **shapes)


def test_peaks_from_unit_counts():
    assert bench.VALU_SLOT_PEAK == 256 * 4 * 16 * 2.4e9          # 39.3 T fp32 lane-ops/s, no packed math
    assert bench.TRANS_PEAK == 256 * 4 * 8 * 2.4e9               # transcendentals at half the fp32 rate
    assert bench.TRANS_SLOTS == 2


def test_ops_of_the_mamba2p8b_layer():
    c = make_config("mamba2p8b_layer")
    ops, trans = bench.algorithmic_ops(c)
    rows = 4 * 2048 * 5120
    # per element: mul, exp2, mul, fma, fma; per (b,d,t): softplus 7 (2 trans), dt*u, D*u, gate 6 (2 trans)
    assert ops == rows * (16 * 5 + 7 + 1 + 1 + 6)
    assert trans == rows * (16 + 4)
    assert bench.valu_slots(ops, trans) == rows * (16 * 6 + 19) == 4823449600


def test_ops_options_and_layouts():
    c = make_config("long_carry")                                 # no gate in this workload
    ops, trans = bench.algorithmic_ops(c)
    rows = 131072 * 2560
    assert ops == rows * (16 * 5 + 7 + 1 + 1) and trans == rows * (16 + 2)
    ops_z, trans_z = bench.algorithmic_ops(c, zoh=True)
    assert ops_z - ops == rows * 16 * bench.ZOH_OPS and trans_z - trans == rows * 16
    ops_c, trans_c = bench.algorithmic_ops(c, conv_k=4)
    assert ops_c - ops == rows * 9 and trans_c - trans == rows * 2
    m = make_config("mamba2_multihead")
    ops, trans = bench.algorithmic_ops(m)
    assert ops == 2 * 8192 * (5120 * (128 * 3 + 2 + 6) + 80 * (7 + 2))
    assert trans == 2 * 8192 * (5120 * 2 + 80 * 3)


def test_ssd_form_flops():
    m = make_config("mamba2_multihead")
    assert round(bench.ssd_form_flops(m) / 1e9, 2) == 59.06


# ---------------------------------------------------------------------------
# bench.py --profile-summary: rocprofv3 CSV -> summary text and traffic record
# ---------------------------------------------------------------------------

_PMC_HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
               '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
               '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
_LIBK = "void ssm::(anonymous namespace)::rowgroup_kernel<ssm::(anonymous namespace)::F32IO, 2, 0, true, false>(ssm::KParams)"


def _pmc_csv(path, rows):
    import os
    os.makedirs(path, exist_ok=True)
    lines = [_PMC_HEADER]
    for i, (kernel, counter, value) in enumerate(rows):
        lines.append(f'{i},{i},"Agent 1",1,1,1,256,7,"{kernel}",256,0,0,32,0,32,"{counter}",{value},0,1')
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def test_profile_summary_from_csv(tmp_path):
    """Synthetic rocprofv3 output with known counts: the traffic record holds the calibrated
    bytes per call (library kernels only, averaged over dispatches), the text the trace and
    the derived SQ figures."""
    import json
    import os
    import subprocess
    import sys
    wl, calib, out = tmp_path / "wl", tmp_path / "calib", tmp_path / "out"
    _pmc_csv(str(calib / "pmc_FETCH_SIZE"), [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 262144.0)])
    _pmc_csv(str(calib / "pmc_WRITE_SIZE"), [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 524288.0)])
    os.makedirs(wl / "trace")
    with open(wl / "trace" / "trace_kernel_stats.csv", "w") as fh:
        fh.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        fh.write(f'"{_LIBK}",25,500000,20000.0,95.0,19000,21000,100.0\n')
        fh.write('"__amd_rocclr_copyBuffer",3,9000,3000.0,5.0,2000,4000,10.0\n')
    _pmc_csv(str(wl / "pmc_FETCH_SIZE"), [(_LIBK, "FETCH_SIZE", 1000.0), (_LIBK, "FETCH_SIZE", 1200.0),
                                          ("void at::native::other_kernel()", "FETCH_SIZE", 99999.0)])
    _pmc_csv(str(wl / "pmc_WRITE_SIZE"), [(_LIBK, "WRITE_SIZE", 500.0)])
    sq = {"SQ_WAVES": 100, "SQ_WAVE_CYCLES": 4000, "SQ_BUSY_CYCLES": 1, "SQ_INSTS_VALU": 1000,
          "SQ_ACTIVE_INST_VALU": 2000, "SQ_INSTS_LDS": 100, "SQ_ACTIVE_INST_LDS": 10, "SQ_WAIT_INST_LDS": 40,
          "SQ_WAIT_INST_ANY": 400, "SQ_INSTS_VALU_TRANS_F32": 100, "SQ_LDS_BANK_CONFLICT": 4, "SQ_INSTS_MFMA": 0,
          "SQ_VALU_MFMA_BUSY_CYCLES": 0, "SQ_INSTS_SALU": 300, "SQ_INSTS_VMEM_RD": 1, "SQ_INSTS_VMEM_WR": 1,
          "GRBM_GUI_ACTIVE": 8 * 40000, "GRBM_COUNT": 8 * 40000, "SQ_WAIT_ANY": 800, "SQ_LDS_ADDR_CONFLICT": 0,
          "SQ_LDS_UNALIGNED_STALL": 0, "SQ_LDS_DATA_FIFO_FULL": 0, "SQ_LDS_CMD_FIFO_FULL": 0, "SQ_INSTS_SMEM": 1,
          "SQ_ACTIVE_INST_ANY": 1, "SQ_ACTIVE_INST_VMEM": 0}
    names = list(sq)
    for i, part in enumerate((names[:8], names[8:18], names[18:])):
        _pmc_csv(str(wl / f"sq{i + 1}"), [(_LIBK, k, sq[k]) for k in part])
    root = os.path.dirname(os.path.abspath(bench.__file__))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--profile-summary", str(wl), "--profile-calib",
                        str(calib), "--profile-tag", "tiny", "--workload", "tiny_f32", "--profile-out", str(out)],
                       capture_output=True, text=True, cwd=root)
    assert r.returncode == 0, r.stderr
    rec = json.load(open(out / "pmc_tiny_f32.json"))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (1100.0 * 2 + 500.0) * 1024      # the other kernel is not the library's
    assert rec["kernel_source_hash"] == bench.kernel_source_hash("tiny_f32")
    assert list(rec["kernel_avg_us"].values()) == [20.0]
    text = open(out / "scan_tiny.txt").read()
    assert "rowgroup_kernel<F32IO, 2, 0, true, false>" in text and "ratio" in text
    sqt = open(out / "sq_counters_tiny.txt").read()
    # 40000 cycles per XCD over a 20 us dispatch = 2.0 GHz; VALU busy = 4 * 2000 / (1024 * 40000)
    assert "2.00 GHz" in sqt and "VALU instructions per wave       10" in sqt
