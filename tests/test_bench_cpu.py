"""CPU checks of bench.py's contract that need no GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode != 0
    assert "one GPU" in proc.stderr


def test_alu_roofline_model():
    # d = 3: ceiling 3.93e13 / 6.5 pairs/s, 10 algorithmic ops per pair
    r = bench.roofline_alu(3, 2.5e9, 2.5e9 / 6.049476923e12)
    assert abs(r["frac"] - 1.0) < 1e-6 and r["ops_per_pair"] == 10 and r["bound"] == "alu"
    assert abs(r["peak"] - 60.495) < 1e-3
    # d = 2: 3.93e13 / 5.5
    assert abs(bench.roofline_alu(2, 1.0, 1.0)["ceiling_pairs_per_s"] - 3.93216e13 / 5.5) < 1e3


def test_mfma_roofline_model():
    r = bench.roofline_mfma(64, 16384.0 ** 2, 16384.0 ** 2 * 128 / 157.3e12)
    assert abs(r["frac"] - 1.0) < 1e-4 and r["bound"] == "mfma" and r["ops_per_pair"] == 128


def test_traffic_record_matches_current_kernels_or_is_absent():
    # a stale record must read as None, never as a number for changed kernels
    for key, fam in (("gmm8_d3_sq:pass", "valu"), ("gauss_d64:pass", "mfma")):
        t = bench.load_traffic(key, fam)
        assert t is None or t > 0


def test_split_roofline_model():
    # the split form: 12 d bf16 flops per pair against 2.5 PFLOP/s, the fp32-equivalent 2 d beside it
    pairs = 16384.0 ** 2
    r = bench.roofline_split(64, pairs, pairs * 768 / 2500e12)
    assert abs(r["frac"] - 1.0) < 1e-4 and r["ops_per_pair"] == 768 and r["bound"] == "mfma"
    assert r["fp32_equivalent"]["ops_per_pair"] == 128
    assert abs(r["fp32_equivalent"]["vs_fp32_mfma_peak"] - 2500.0 / 6 / 157.3) < 1e-3
    assert [bench.packed_stride(d) for d in (9, 16, 17, 32, 33, 64, 65, 256)] == [16, 16, 32, 32, 64, 64, 128, 256]


def test_inputs_dimension_override():
    from sk_inputs import make_inputs

    x, y, a, b = make_inputs("gauss_d64", n=40, m=30, d=24)
    assert x.shape == (40, 24) and y.shape == (30, 24) and a.shape == (40,) and b.shape == (30,)
    x2, _, _, _ = make_inputs("gauss_d64", n=40, m=30, d=24)
    assert (x == x2).all()  # seeded
    x64, _, _, _ = make_inputs("gauss_d64", n=40, m=30)
    assert x64.shape == (40, 64)
