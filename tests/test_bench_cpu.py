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
