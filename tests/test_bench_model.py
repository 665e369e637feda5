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
