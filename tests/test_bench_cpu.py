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
    # d = 3: ceiling 3.93e13 / 5.5 pairs/s (the exp2 issues beside the 5.5 other slots); the peak is the chip's
    # lane-slot rate, 256 x 4 x 16 x 2.4e9
    ceil3 = 256 * 4 * 16 * 2.4e9 / 5.5
    r = bench.roofline_alu(3, 2.5e9, 2.5e9 / ceil3)
    assert abs(r["frac"] - 1.0) < 1e-6 and r["slots_per_pair"] == 5.5 and r["bound"] == "alu"
    assert abs(r["peak"] - 256 * 4 * 16 * 2.4e9 / 1e12) < 1e-3 and r["unit"] == "T VALU lane-slots/s"
    # the same launch in fp32 flops: 2d + 3 = 9 per pair against the published 157.3 and 78.6 TFLOP/s
    assert r["fp32_flops_per_pair"] == 9
    tflops = ceil3 * 9 / 1e12
    assert abs(r["fp32_tflops"] - tflops) < 1e-3
    assert abs(r["frac_fp32_peak"] - tflops / 157.3) < 1e-4 and abs(r["frac_fp32_nonpacked"] - tflops / 78.6) < 1e-4
    # the pass of the 50k x 50k workload at its measured 434.71 us: 0.33 of 157.3, 0.66 of 78.6
    r = bench.roofline_alu(3, 2.5e9, 434.71e-6)
    assert abs(r["frac_fp32_peak"] - 0.329) < 1e-3 and abs(r["frac_fp32_nonpacked"] - 0.6585) < 1e-3
    # d = 2: 3.93e13 / 4.5; a 4-column payload adds 4 slots
    assert abs(bench.roofline_alu(2, 1.0, 1.0)["ceiling_pairs_per_s"] - 3.93216e13 / 4.5) < 1e3
    assert abs(bench.roofline_alu(3, 1.0, 1.0, 4)["ceiling_pairs_per_s"] - 3.93216e13 / 9.5) < 1e3


def test_mfma_roofline_model():
    r = bench.roofline_mfma(64, 16384.0 ** 2, 16384.0 ** 2 * 128 / 157.3e12)
    assert abs(r["frac"] - 1.0) < 1e-4 and r["bound"] == "mfma" and r["ops_per_pair"] == 128


def test_traffic_record_matches_current_kernels_or_is_absent():
    # a stale record must read as None, never as a number for changed kernels
    for key, fam, kernel in (("gmm8_d3_sq:pass", "valu", "k_pass_valu<3>"),
                             ("gauss_d64:pass", "mfma", "k_pass_mfma<64>")):
        t = bench.load_traffic(key, fam, kernel)
        assert t is None or t > 0
        # the record of a pass is never reported for another kernel of the same workload (a transport launch)
        assert bench.load_traffic(key, fam, "k_transport_mfma<64,1,4>") is None


def test_split_roofline_model():
    # the split form: 6 d fp16 flops per pair (three products) against 2.5 PFLOP/s, 8 d at a padded width of
    # 16 (four products in two instructions); the fp32-equivalent 2 d beside it
    pairs = 16384.0 ** 2
    r = bench.roofline_split(64, pairs, pairs * 384 / 2500e12)
    assert abs(r["frac"] - 1.0) < 1e-4 and r["ops_per_pair"] == 384 and r["bound"] == "mfma"
    assert r["fp32_equivalent"]["ops_per_pair"] == 128
    assert abs(r["fp32_equivalent"]["vs_fp32_mfma_peak"] - 2500.0 / 3 / 157.3) < 1e-3
    assert bench.roofline_split(12, pairs, 1.0)["ops_per_pair"] == 96
    assert bench.roofline_split(17, pairs, 1.0)["ops_per_pair"] == 102
    assert [bench.packed_stride(d) for d in (9, 16, 17, 32, 33, 64, 65, 256)] == [16, 16, 32, 32, 64, 64, 128, 256]


def test_transport_split_roofline_model():
    # fp16 split scores (6 d) and fp32 weighted sums (2 per padded payload column) share the matrix pipe: at
    # d = 64 with 64 columns one pair needs 384 / 2500e12 + 128 / 157.3e12 s of it
    pairs = 16384.0 ** 2
    pipe = 384 / 2500e12 + 128 / 157.3e12
    r = bench.roofline_transport_split(64, pairs, pairs * pipe, 64)
    assert abs(r["frac"] - 1.0) < 1e-3 and r["ops_per_pair"] == 256 and r["bound"] == "mfma"
    assert abs(r["peak"] - 256 / pipe / 1e12) < 1e-2
    # a launch of 20 columns runs a 64-column tile; one of 9 a 16-column tile
    r20 = bench.roofline_transport_split(33, pairs, 1.0, 20)
    assert r20["ops_per_pair"] == 2 * 33 + 40 and "weighted sums (128)" in r20["mfma_dtype"]
    # the gradient (transport mode 4): the weighted key sums run over all P = 128 padded coordinates
    # the gradient up to a padded width of 64: the weighted sums as three fp16 products too, 6 flops per column
    rs = bench.roofline_transport_split(64, pairs, pairs * (384 + 384) / 2500e12, 64, cols=64, split_sums=True)
    assert abs(rs["frac"] - 1.0) < 1e-3 and "fp16 split weighted sums (384)" in rs["mfma_dtype"]
    rg = bench.roofline_transport_split(100, pairs, 1.0, 100, cols=128)
    assert rg["ops_per_pair"] == 400 and "weighted sums (256)" in rg["mfma_dtype"]
    r9 = bench.roofline_transport_split(12, pairs, 1.0, 9)
    assert r9["ops_per_pair"] == 2 * 12 + 18 and "(96 flops per pair)" in r9["mfma_dtype"]
    assert "weighted sums (32)" in r9["mfma_dtype"]


def test_inputs_dimension_override():
    from sk_inputs import make_inputs

    x, y, a, b = make_inputs("gauss_d64", n=40, m=30, d=24)
    assert x.shape == (40, 24) and y.shape == (30, 24) and a.shape == (40,) and b.shape == (30,)
    x2, _, _, _ = make_inputs("gauss_d64", n=40, m=30, d=24)
    assert (x == x2).all()  # seeded
    x64, _, _, _ = make_inputs("gauss_d64", n=40, m=30)
    assert x64.shape == (40, 64)


def test_record_traffic_from_counter_csv(tmp_path, monkeypatch):
    # two rocprofv3-style counter CSVs: the pass launched twice, one 256 MiB calibration copy and a small copy
    header = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"

    def write(run, counter, copy_kib, pass_kib):
        d = tmp_path / run / "host" / "123"
        d.mkdir(parents=True)
        rows = [f'1,"__amd_rocclr_copyBuffer",{counter},40.0',
                f'2,"__amd_rocclr_copyBuffer",{counter},{copy_kib}',
                f'3,"void sk::(anonymous namespace)::k_pass_valu<3>(sk::PassArgs)",{counter},{pass_kib[0]}',
                f'4,"void sk::(anonymous namespace)::k_merge(sk::PassArgs)",{counter},999.0',
                f'5,"void sk::(anonymous namespace)::k_pass_valu<3>(sk::PassArgs)",{counter},{pass_kib[1]}']
        (d / "p_counter_collection.csv").write_text(header + "\n".join(rows) + "\n")
        return str(tmp_path / run)

    fetch_dir = write("fetch", "FETCH_SIZE", 131072.0, (3000.0, 3200.0))  # FETCH reads half the true bytes
    write_dir = write("write", "WRITE_SIZE", 262144.0, (6400.0, 6400.0))
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    e = bench.record_traffic("w:pass", "k_pass_valu<3>", "valu", fetch_dir, write_dir, 256)
    assert e["fetch_factor"] == 0.5 and e["write_factor"] == 1.0
    assert e["fetch_kib_raw"] == 3100.0 and e["write_kib_raw"] == 6400.0
    assert e["bytes_per_launch"] == (6200.0 + 6400.0) * 1024.0
    # the record is read back while the kernel's sources hash the same
    assert bench.load_traffic("w:pass", "valu", "k_pass_valu<3>") == e["bytes_per_launch"]
    assert bench.load_traffic("w:pass", "mfma", "k_pass_valu<3>") is None
