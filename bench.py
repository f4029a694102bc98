#!/usr/bin/env python3
"""Throughput of the streamed log-domain Sinkhorn hot path on one MI355X.

One step = the whole hot path over one synthetic problem already resident in
HBM: sk_solve (centre + pack, n_iters alternating row/column streamed passes
with the fused marginal-residual check every `check_every` iterations),
sk_cost and sk_grad_x.  The default workload is the throughput headline:
n = m = 50,000 points in 3-D drawn from 8-Gaussian mixtures in the unit cube,
Exponential(1) weights, eps = 0.01, 100 iterations.

Printed (one JSON line):
  value        point-pair evaluations per second, counting the 2 n m n_iters
               evaluations of the Sinkhorn iterations only (the residual probe
               and gradient passes are done inside the timed step but not
               counted), over the wall-clock of the timed steps;
  roofline     the streamed-pass kernel (the dominant kernel, timed live with
               HIP events on the launch stream around every --timing-stride-th
               pass launch of the timed steps) against the vector-ALU issue
               ceiling of the chip in lane-slots/s, with its fp32 flop rate
               against the published fp32 vector peaks beside it (see
               roofline_alu);
  components_ms  each part of the step timed on its own after the timed
               steps (median of 3): the solve alone, the cost, the gradient
               and the standalone two-pass marginal residual, with the solve's
               own pair-evals/s and iterations/s beside them;
  cpu_baseline the CPU oracle as it stands, timed on alternating iterations
               of the same workload on this host (about 10 s of them);
  extra        {"configs": [...]}: after the headline, one line per other
               workload (EXTRA_CONFIGS), each timed the same way -- value,
               iterations/s and the roofline of its pass kernel: the 1000-point,
               10k^2 and d = 64 problems as HIP-graph replays (their passes
               are short enough for launch gaps to show), the 50k x 40k problem
               eagerly, and 2 of the 50 iterations of the 2^20-point problem.

Other steps (--mode, same workload and JSON fields; value counts the pair
evaluations of the counted iterations only):
  symmetric   sk_solve_ex, symmetric (Jacobi) variant with blend --alpha,
              fixed n_iters, then the general dual cost sk_dual_cost;
  marginal,   sk_solve_ex, alternating, stop rule with --stop-tol, cap n_iters,
  potential   check every --check-every; the line adds iters_run, converged,
              final_viol and the time of a fixed run of iters_run iterations
              (the stop rule's overhead);
  divergence  sk_divergence, n_iters per term: 2 n_iters (n m + n^2 + m^2)
              pair evaluations;
  flow        one step of the gradient flow (sk_gradient_flow with one step:
              fresh solve of n_iters iterations, cost, gradient, x <- x - lr
              grad, x updated in place); --graph replays it as a HIP graph;
  hvp         one Hessian-vector product sk_hvp with --cg-iters conjugate-
              gradient steps at the potentials of an n_iters solve done
              before timing: (3 + 2 cg_iters) n m pair evaluations;
  transport   one transport product P Y~-sized: sk_transport with a k = d
              payload (the barycentric numerator), n m pair evaluations.
  grad        one sk_grad_x at the potentials of an n_iters solve done
              before timing: n m pair evaluations, twice that for d > 8
              (a store-lse pass, then the weighted key sums), whose roofline
              the line reports.
  fs2         the two-stage block-sparse solver sk_fs2_solve to a marginal
              target of --fs2-tol-rel times the largest point mass; value
              counts the dense-equivalent 2 n m evaluations per fine
              iteration; the line adds the solver's counts, the kept fraction,
              the time of the ordering, coarse stage and lift alone (a run
              with no fine iteration, untimed), the all-particle residual of
              the result (two dense passes, up to n m = 2e14) and,
              with --fs2-dense, the time of the dense solver (stop rule
              "marginal", same tolerance) for the same problem.
The roofline of the hvp / transport modes is that of the transport kernel
(the dominant one) with its payload work per pair; that of the fs2 mode is the
block-sparse pass of the fine stage, counting the point pairs of the kept tiles
(its iters_per_s counts fine iterations).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X unit counts and clock: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz.
CUS, SIMDS, LANES, CLOCK_HZ = 256, 4, 16, 2.4e9
LANE_OPS_PER_S = CUS * SIMDS * LANES * CLOCK_HZ  # 3.93e13 single-lane VALU ops / s (no packed fp32)
# Issue model of the vector ALUs on gfx950, from the issue-rate micro-benchmarks
# (`python bench.py --ceilings`) and the SQ counters of the pass kernels: every
# non-transcendental VALU instruction (FMA, add, subtract, multiply, max) takes
# one issue slot, a wave64 instruction every 4 cycles on a 16-lane SIMD, and
# independent chains of them reach 0.98 of that rate.  v_exp_f32 runs on the
# transcendental unit at half the lane rate; in the pass it issues beside the
# other instructions (at 2^20 points the pass issues 1.07x the single-issue
# limit when the exp2 are counted as slots, 0.89x without them), so the
# ceiling counts the non-transcendental slots and checks the exp2 rate apart.
EXP_RATE_FRACTION = 0.5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pass_traffic.json")


FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak (packed fp32: two lanes' FMAs per slot)
FP32_NONPACKED_PEAK_TFLOPS = 78.6  # the same units issuing one fp32 FMA per lane per cycle


def roofline_alu(d: int, pairs_per_launch: float, avg_launch_s: float, payload: int = 0) -> dict:
    """Vector-ALU roofline of one streamed pass.

    The pass is bound by vector instruction issue.  Fewest non-transcendental
    issue slots per pair evaluation: d FMAs (the bias rides in the first FMA's
    addend), 1/2 for the running max (v_max3 takes two new scores per
    instruction), one subtract and one add: d + 2.5 lane-slots; the pair's
    exp2 runs on the transcendental unit beside them.  The chip issues
    LANE_OPS_PER_S = 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13 lane-slots
    per second, the exp2 unit completing at half that rate, so the ceiling is
    min(LANE_OPS_PER_S / (d + 2.5), EXP_RATE_FRACTION * LANE_OPS_PER_S) pairs/s.
    `achieved`, `peak` and `frac` are in lane-slots per second: the minimal
    slots of the pairs evaluated per launch over the launch duration, against
    the slots the chip can issue (capped by the exp2 rate).

    The same launch is also priced in fp32 flops against the chip's published
    fp32 vector peaks: 2d + 3 flops per pair (d FMAs, the max, the subtract and
    the add; the exp2 is a transcendental, not a flop), over 157.3 TFLOP/s
    (packed fp32) and 78.6 TFLOP/s (one FMA per lane per cycle).  A transport
    pass with a payload of K columns adds K FMAs per pair (K slots, 2K flops).
    """
    slots_per_pair = d + 2.5 + payload
    ceiling_pairs = min(LANE_OPS_PER_S / slots_per_pair, EXP_RATE_FRACTION * LANE_OPS_PER_S)
    achieved = pairs_per_launch * slots_per_pair / avg_launch_s / 1e12
    peak = ceiling_pairs * slots_per_pair / 1e12
    flops_per_pair = 2 * d + 3 + 2 * payload
    tflops = pairs_per_launch * flops_per_pair / avg_launch_s / 1e12
    return {"bound": "alu", "achieved": round(achieved, 3), "peak": round(peak, 3),
            "unit": "T VALU lane-slots/s", "frac": round(achieved / peak, 4), "traffic": None,
            "slots_per_pair": slots_per_pair, "fp32_flops_per_pair": flops_per_pair,
            "fp32_tflops": round(tflops, 3),
            "frac_fp32_peak": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
            "frac_fp32_nonpacked": round(tflops / FP32_NONPACKED_PEAK_TFLOPS, 4),
            "pairs_per_launch": pairs_per_launch,
            "avg_launch_us": round(avg_launch_s * 1e6, 3), "ceiling_pairs_per_s": ceiling_pairs}


MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak (the same rate as bf16)


def roofline_mfma(d: int, pairs_per_launch: float, avg_launch_s: float, payload: int = 0) -> dict:
    """Matrix-core roofline of one streamed pass for d > 8: the algorithmic work is
    the cross term, 2d flops per pair evaluation (plus 2 per payload column of a
    transport pass), against the fp32 MFMA peak."""
    ops = 2 * d + 2 * payload
    achieved = pairs_per_launch * ops / avg_launch_s / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4), "traffic": None, "ops_per_pair": ops,
            "pairs_per_launch": pairs_per_launch, "avg_launch_us": round(avg_launch_s * 1e6, 3)}


def packed_stride(d: int) -> int:
    """The library's padded dimension of the matrix-core layout (d > 8)."""
    return max(16, 1 << (d - 1).bit_length())


def roofline_split(d: int, pairs_per_launch: float, avg_launch_s: float) -> dict:
    """Matrix-core roofline of the solver pass (and the one-column transport kernel), where the cross term
    runs on fp16 matrix instructions from a scaled two-part split of each coordinate: three products
    (6 d fp16 flops per pair evaluation) from 32 padded coordinates on, four in two instructions at a
    padded width of 16 (8 d), against the dense fp16 MFMA peak. The fp32-equivalent rate (2 d flops per
    pair, the fp32 contraction it replaces) is reported beside it."""
    ops = (8 if packed_stride(d) == 16 else 6) * d
    achieved = pairs_per_launch * ops / avg_launch_s / 1e12
    fp32_eq = pairs_per_launch * 2 * d / avg_launch_s / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None, "ops_per_pair": ops,
            "mfma_dtype": "fp16 (scaled two-part split of fp32: hh + hl + lh)",
            "fp32_equivalent": {"achieved": round(fp32_eq, 3), "ops_per_pair": 2 * d,
                                "vs_fp32_mfma_peak": round(fp32_eq / MFMA_FP32_PEAK_TFLOPS, 4)},
            "pairs_per_launch": pairs_per_launch, "avg_launch_us": round(avg_launch_s * 1e6, 3)}


def roofline_transport_split(d: int, pairs_per_launch: float, avg_launch_s: float, payload: int,
                             cols: int | None = None, split_sums: bool = False) -> dict:
    """Matrix-core roofline of one transport-product launch for d > 8 carrying `payload` columns (at most the
    library's chunk: 64 from a padded width of 64, else 16): the scores in the fp16 split form (6 d fp16 flops
    per pair, 8 d at a padded width of 16) and the weighted sums on fp32 matrix instructions (2 per column of
    the launch's 16- or 64-column tile). The ceiling is the time the matrix pipe needs for both at their own
    dense peaks; `achieved` and `peak` are stated in the method's flops per pair (2 d + 2 x payload), `peak`
    being the rate that pipe time allows. `cols` overrides the tile width (the gradient's weighted key sums
    run over all P padded coordinates). `split_sums`: the weighted sums run on fp16 matrix instructions as three
    products of two-part splits (6 fp16 flops per pair and column; modes 0, 1 and 4 up to a padded width of 128)."""
    f16_ops = (8 if packed_stride(d) == 16 else 6) * d
    if cols is None:
        cols = 16 if payload <= 16 else 64
    if split_sums:
        pipe_s_per_pair = (f16_ops + 6 * cols) / (MFMA_F16_PEAK_TFLOPS * 1e12)
        sums = "fp16 split weighted sums (%d)" % (6 * cols)
    else:
        pipe_s_per_pair = f16_ops / (MFMA_F16_PEAK_TFLOPS * 1e12) + 2 * cols / (MFMA_FP32_PEAK_TFLOPS * 1e12)
        sums = "fp32 weighted sums (%d)" % (2 * cols)
    ops = 2 * d + 2 * payload
    achieved = pairs_per_launch * ops / avg_launch_s / 1e12
    peak = ops / pipe_s_per_pair / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 3), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None, "ops_per_pair": ops,
            "mfma_dtype": "fp16 split scores (%d flops per pair), %s" % (f16_ops, sums),
            "fp32_equivalent": {"achieved": round(achieved, 3), "ops_per_pair": ops,
                                "vs_fp32_mfma_peak": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4)},
            "pairs_per_launch": pairs_per_launch, "avg_launch_us": round(avg_launch_s * 1e6, 3)}


# Sources that determine each timed kernel's code (plus the device flags).
KERNEL_SOURCES = {
    "valu": ["sk_pass_valu.hip", "sk_pass_common.hpp", "sk_internal.hpp"],
    "mfma": ["sk_pass_mfma.hip", "sk_pass_common.hpp", "sk_internal.hpp"],
}


def kernel_source_hash(family: str) -> str:
    import hashlib

    from streaming_sinkhorn_solver_amd import build as skbuild

    h = hashlib.sha256(" ".join(skbuild.DEVICE_FLAGS).encode())
    for name in KERNEL_SOURCES[family]:
        h.update(open(os.path.join(skbuild.CSRC, name), "rb").read())
    return h.hexdigest()


def load_traffic(kernel_key: str, family: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken of this kernel, on its current source (else None)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(kernel_key)
    if not entry or entry.get("kernel") != kernel or entry.get("source_sha256") != kernel_source_hash(family):
        return None
    return entry.get("bytes_per_launch")


def counter_per_launch(run_dir: str, counter: str, kernel_pattern: str, largest: bool = False) -> float:
    """KiB per dispatch of one rocprofv3 --pmc counter for the kernels whose name
    contains kernel_pattern, averaged over their dispatches (or the largest
    dispatch, for the calibration copy), from the CSV files under run_dir."""
    import csv
    import glob

    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter or kernel_pattern not in row.get("Kernel_Name", ""):
                    continue
                key = (path, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} records of a kernel named like {kernel_pattern!r} under {run_dir}")
    vals = list(per.values())
    return max(vals) if largest else sum(vals) / len(vals)


def record_traffic(key: str, kernel: str, family: str, fetch_dir: str, write_dir: str, copy_mib: int) -> dict:
    """Writes the calibrated HBM bytes per launch of `kernel` into the traffic
    record: FETCH_SIZE and WRITE_SIZE (KiB, separate runs of bench.py with
    --copy-calibration copy_mib under rocprofv3 --pmc), each divided by what the
    same counter reads for the copy of known size in the same run."""
    pattern = kernel + "("
    true_kib = copy_mib * 1024.0
    fetch = counter_per_launch(fetch_dir, "FETCH_SIZE", pattern)
    write = counter_per_launch(write_dir, "WRITE_SIZE", pattern)
    fetch_factor = counter_per_launch(fetch_dir, "FETCH_SIZE", "copyBuffer", largest=True) / true_kib
    write_factor = counter_per_launch(write_dir, "WRITE_SIZE", "copyBuffer", largest=True) / true_kib
    entry = {"kernel": kernel,
             "bytes_per_launch": (fetch / fetch_factor + write / write_factor) * 1024.0,
             "fetch_kib_raw": fetch, "write_kib_raw": write,
             "fetch_factor": fetch_factor, "write_factor": write_factor,
             "source_sha256": kernel_source_hash(family), "sources": KERNEL_SOURCES[family]}
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    rec[key] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return entry


def run_ceilings():
    import ctypes

    import torch

    from streaming_sinkhorn_solver_amd import build as skbuild

    lib = ctypes.CDLL(skbuild.UBENCH_PATH)
    lib.sku_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 2048 * 4, 2000
    out = torch.empty(blocks * 256, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for kind, name in ((0, "fma"), (1, "exp2"), (2, "pair_mix_d3"), (3, "mfma_f32_16x16x4"), (4, "mfma_f32_32x32x2"),
                       (5, "mfma_f32_16x16x32_bf16"), (6, "mfma_bf16_with_8_fma")):
        for _ in range(2):
            lib.sku_launch(kind, blocks, 50, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.sku_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0, rc
        secs = e0.elapsed_time(e1) * 1e-3
        if kind <= 2:
            rate = blocks * 256 * iters * 64 / secs
            res[name] = {"ops_per_s": rate, "frac_of_lane_rate": rate / LANE_OPS_PER_S}
        elif kind <= 4:
            flops = blocks * 4 * iters * 64 * (2048 if kind == 3 else 4096)
            res[name] = {"tflops": flops / secs / 1e12, "frac_of_peak": flops / secs / 1e12 / MFMA_FP32_PEAK_TFLOPS}
        else:
            flops = blocks * 4 * iters * 64 * 16384
            res[name] = {"tflops": flops / secs / 1e12, "frac_of_peak": flops / secs / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "ms": secs * 1e3}
    # SIMD cycles per bf16 matrix instruction, alone and with 8 wave-wide FMAs (32 cycles at 16 lanes per cycle)
    insts_per_simd = blocks * 4 / (CUS * SIMDS) * iters * 64
    for key, name in (("bf16_mfma_cycles", "mfma_f32_16x16x32_bf16"), ("bf16_mfma_plus_8fma_cycles",
                                                                      "mfma_bf16_with_8_fma")):
        res[key] = res[name]["ms"] * 1e-3 * CLOCK_HZ / insts_per_simd
    res["exp2_issue_cost"] = res["fma"]["ops_per_s"] / res["exp2"]["ops_per_s"]
    # fp16 matrix instructions with vector work beside each: SIMD cycles per matrix instruction
    f16 = {}
    for kind, name in ((19, "f16_alone"), (20, "f16+8fma"), (21, "f16+4exp"), (22, "f16+3fma+1exp"),
                       (23, "f16+3fma+1exp_on_results"), (24, "f16+3fma_on_results")):
        for _ in range(2):
            lib.sku_launch(kind, blocks, 50, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.sku_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0, rc
        secs = e0.elapsed_time(e1) * 1e-3
        f16[name] = {"ms": secs * 1e3, "cycles_per_mfma": secs * CLOCK_HZ / insts_per_simd}
    res["f16_mfma_mix"] = f16
    # does v_exp_f32 take an issue slot beside FMAs?  NF FMAs + NE exp2 per chain step: times of one launch
    mix = {}
    for kind, nf, ne in ((7, 6, 0), (8, 6, 1), (9, 7, 0), (10, 4, 1), (11, 2, 1), (12, 6, 1), (13, 2, 1), (14, 6, 1),
                         (15, 6, 0), (16, 6, 0), (17, 6, 0)):
        for _ in range(2):
            lib.sku_launch(kind, blocks, 50, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.sku_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        assert rc == 0, rc
        secs = e0.elapsed_time(e1) * 1e-3
        steps = blocks * 256 * iters * 64 / secs  # chain steps per second, lane-wise
        name = {15: "6add", 16: "6sub", 17: "6mul"}.get(kind, f"{nf}fma+{ne}exp" + (
            "_interleaved" if kind == 14 else "_plain" if kind >= 12 else "_neg"))
        mix[name] = {"ms": secs * 1e3, "fma_lane_ops_per_s": steps * nf,
                                   "fma_slots_per_step": mix_fma_rate / steps if kind != 7 else float(nf)}
        if kind == 7:
            mix_fma_rate = steps * nf  # FMA lane-ops/s with independent chains, no exp2
    res["fma_exp_mix"] = mix
    # device-wide barrier of a cooperative launch: microseconds per grid.sync() at a few grid sizes
    gs = {}
    for nb in (8, 64, 256, 512):
        rc = lib.sku_launch(18, nb, 10, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        if rc != 0:
            gs[nb] = f"launch refused ({rc})"
            continue
        times = []
        for it in (100, 1100):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.sku_launch(18, nb, it, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        gs[nb] = {"us_per_sync": (times[1] - times[0]) / 1000.0, "launch_us_100": times[0]}
    res["grid_sync"] = gs
    res["lane_ops_per_s_nominal"] = LANE_OPS_PER_S
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="gmm8_d3_sq")
    ap.add_argument("--iters", type=int, default=None, help="override the workload's iteration count")
    ap.add_argument("--size", type=int, default=None, help="override n = m (same recipe, e.g. a smaller problem)")
    ap.add_argument("--dim", type=int, default=None, help="override d (same recipe in d dimensions)")
    ap.add_argument("--eps-blur", action="store_true",
                    help="eps = n^(-2/3), the squared mean spacing of n points in the unit cube (the cluster_d3 "
                         "workload's rule) at the --size given")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the other workloads the default run times after the headline")
    ap.add_argument("--ceilings", action="store_true", help="run the issue-rate micro-benchmarks and exit")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time its replays (kernel timing from an eager step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device (a known-size reference for HBM byte counters)")
    ap.add_argument("--timing-stride", type=int, default=7,
                    help="time every k-th pass launch with HIP events (odd, so row and column passes alternate)")
    ap.add_argument("--mode", default="solve",
                    choices=["solve", "symmetric", "marginal", "potential", "divergence", "flow", "hvp", "transport", "grad",
                             "fs2", "primal"])
    ap.add_argument("--fs2-block", type=int, default=512)
    ap.add_argument("--fs2-tol-rel", type=float, default=0.01, help="target residual / largest point mass")
    ap.add_argument("--fs2-delta", type=float, default=1e-6)
    ap.add_argument("--fs2-max-iters", type=int, default=5000)
    ap.add_argument("--fs2-dense", action="store_true", help="also time the dense solver to the same tolerance")
    ap.add_argument("--cg-iters", type=int, default=20, help="conjugate-gradient steps of the hvp mode")
    ap.add_argument("--lr", type=float, default=0.1, help="step size of the gradient flow")
    ap.add_argument("--alpha", type=float, default=0.5, help="blend of the symmetric variant")
    ap.add_argument("--stop-tol", type=float, default=1e-5, help="tolerance of the marginal / potential stop rule")
    ap.add_argument("--check-every", type=int, default=10, help="check interval of the stop rules")
    ap.add_argument("--record-traffic", nargs=4, metavar=("KEY", "FAMILY", "FETCH_DIR", "WRITE_DIR"),
                    help="write the calibrated HBM bytes per launch of the workload's dominant pass kernel (FAMILY "
                         "valu or mfma) from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into the traffic "
                         "record under KEY, and exit (no GPU use; needs --copy-calibration and --dim as in the runs)")
    args = ap.parse_args()

    if args.record_traffic:
        key, family, fetch_dir, write_dir = args.record_traffic
        if not args.copy_calibration:
            sys.exit("--record-traffic needs --copy-calibration MIB, the size the runs copied")
        from sk_inputs import WORKLOADS

        d = args.dim or WORKLOADS[args.workload].d
        kernel = f"k_pass_valu<{d}>" if family == "valu" else f"k_pass_mfma<{packed_stride(d)}>"
        print(json.dumps(record_traffic(key, kernel, family, fetch_dir, write_dir, args.copy_calibration)))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d); run it with --gpus 1." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import streaming_sinkhorn_solver_amd as sk
    from sk_inputs import WORKLOADS, eps32, make_inputs

    if args.ceilings:
        run_ceilings()
        return

    if args.graph and args.mode in ("marginal", "potential"):
        print("a stop rule synchronises at every check and cannot be captured: drop --graph", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    n_iters = w.n_iters if args.iters is None else args.iters
    eps = eps32(w.eps)
    x, y, a, b = make_inputs(args.workload, n=args.size, m=args.size, d=args.dim)
    print(f"inputs ready: {x.shape[0]} x {y.shape[0]}, d = {x.shape[1]}", file=sys.stderr, flush=True)
    if args.eps_blur:
        eps = eps32(float(x.shape[0]) ** (-2.0 / 3.0))
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    dev = torch.device("cuda:0")
    X, Y, A, B = (torch.from_numpy(v).to(dev) for v in (x, y, a, b))
    ws = sk.workspace(n, m, d, dev)
    f = torch.empty(n, dtype=torch.float32, device=dev)
    g = torch.empty(m, dtype=torch.float32, device=dev)
    ce = w.check_every
    trace = torch.empty(max(n_iters // ce, 1) if ce else 1, dtype=torch.float32, device=dev)
    cost_out = torch.empty(1, dtype=torch.float64, device=dev)
    grad = torch.empty((n, d), dtype=torch.float32, device=dev)
    sk.check_inputs(X, Y, A, B, ws)  # data validation once, outside the timed region
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: {args.copy_calibration} MiB read + {args.copy_calibration} MiB written",
              file=sys.stderr)
        del src, dst

    mode = args.mode
    stop = {}
    fs2_info = {}
    if mode == "fs2":
        fs2_tol = args.fs2_tol_rel * float(max(A.max().item(), B.max().item()))
        nb = sk.load_library().sk_fs2_workspace_bytes(n, m, d, args.fs2_block, 1024)
        ws_fs2 = torch.empty(nb, dtype=torch.uint8, device=dev)
    if mode in ("hvp", "transport", "grad", "primal"):
        # potentials of a full solve, outside the timed region
        sk.solve(X, Y, A, B, eps=eps, n_iters=n_iters, ws=ws, f=f, g=g, check=False)
        ws_t = sk.transport_workspace(n, m, d, dev)
        v_dir = torch.randn((n, d), generator=torch.Generator(device="cpu").manual_seed(7)).to(dev)
        hv_out = torch.empty((n, d), dtype=torch.float32, device=dev)
        cg_res = torch.empty(1, dtype=torch.float32, device=dev)
        y_pay = Y.contiguous()
    dv_out = torch.empty(4, dtype=torch.float64, device=dev)
    primal_out = torch.empty(2, dtype=torch.float64, device=dev)
    ws_div = sk.divergence_workspace(n, m, d, dev) if mode == "divergence" else None

    def step():
        if mode == "solve":
            sk.solve(X, Y, A, B, eps=eps, n_iters=n_iters, check_every=ce, ws=ws, f=f, g=g, trace=trace, check=False)
            sk.cost(A, B, f, g, eps=eps, out=cost_out)
            if w.grad:
                sk.grad_x(X, Y, A, B, g, eps=eps, ws=ws, out=grad)
        elif mode == "symmetric":
            sk.solve_ex(X, Y, A, B, eps=eps, variant="symmetric", alpha=args.alpha, max_iter=n_iters, ws=ws, f=f,
                        g=g, check=False)
            sk.dual_cost(X, Y, A, B, f, g, eps=eps, ws=ws, out=cost_out)
        elif mode in ("marginal", "potential"):
            _, _, it, conv, viol = sk.solve_ex(X, Y, A, B, eps=eps, stop_mode=mode, stop_tol=args.stop_tol,
                                               max_iter=n_iters, check_every=args.check_every, ws=ws, f=f, g=g,
                                               check=False)
            stop.update(iters_run=it, converged=conv, final_viol=viol)
            sk.cost(A, B, f, g, eps=eps, out=cost_out)
        elif mode == "hvp":
            sk.hvp(X, Y, A, B, f, g, v_dir, eps=eps, cg_iters=args.cg_iters, ws=ws_t, out=hv_out, cg_resid=cg_res)
        elif mode == "transport":
            sk.transport(X, Y, A, B, f, g, y_pay, eps=eps, ws=ws_t, out=hv_out)
        elif mode == "grad":
            sk.grad_x(X, Y, A, B, g, eps=eps, ws=ws, out=grad)
        elif mode == "primal":
            sk.primal_cost(X, Y, A, B, f, g, eps=eps, ws=ws_t, out=primal_out)
        elif mode == "fs2":
            _, _, inf = sk.fs2_solve(X, Y, A, B, eps=eps, block=args.fs2_block, tol=fs2_tol, delta=args.fs2_delta,
                                     max_iters=args.fs2_max_iters, ws=ws_fs2, f=f, g=g, check=False)
            fs2_info.update(inf)
        elif mode == "flow":
            sk.gradient_flow(X, Y, A, B, eps=eps, n_iters=n_iters, n_steps=1, lr=args.lr, ws=ws, f=f, g=g,
                             grad=grad, cost_trace=cost_out, check=False)
        else:
            sk.divergence(X, Y, A, B, eps=eps, n_iters=n_iters, ws=ws_div, out=dv_out, check=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # pass-kernel durations from one eager step; the timed steps replay the graph
        sk.timing_enable(True, args.timing_stride)
        step()
        torch.cuda.synchronize()
        pass_ms, launches, pairs = sk.timing_read()
        sk.timing_enable(False)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    else:
        sk.timing_enable(True, args.timing_stride)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        graph.replay() if graph is not None else step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if graph is None:
        pass_ms, launches, pairs = sk.timing_read()
        sk.timing_enable(False)

    wall_s = t1 - t0
    print(f"timed steps done: {wall_s:.3f} s", file=sys.stderr, flush=True)
    gpu_s = ev0.elapsed_time(ev1) * 1e-3
    step_s = max(wall_s, gpu_s) / args.steps
    counted_iters = stop.get("iters_run", n_iters)
    pair_evals = 2.0 * n * m * counted_iters
    if mode == "divergence":
        pair_evals = 2.0 * n_iters * (n * m + n * n + m * m)
    if mode == "hvp":
        pair_evals = (3.0 + 2.0 * args.cg_iters) * n * m
    if mode == "transport":
        pair_evals = 1.0 * n * m
    if mode == "grad":
        pair_evals = (2.0 if d > 8 else 1.0) * n * m
    if mode == "primal":
        pair_evals = (3.0 if d > 8 else 2.0) * n * m  # (d > 8: the store-lse pass,) the weighted row pass, the column pass  # d > 8: the store-lse pass, then the weighted sums
    if mode == "fs2":
        pair_evals = 2.0 * n * m * fs2_info["fine_iters"]
    extra = {}
    if mode == "solve":
        # each part of the step on its own (outside the timed steps; median of 3, HIP events on the stream
        # the library launches on): the solve alone (prep + K iterations + fused residuals), the cost, the
        # gradient and the standalone two-pass marginal residual
        def part_ms(fn):
            times = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            return sorted(times)[1]

        parts = {
            "solve": part_ms(lambda: sk.solve(X, Y, A, B, eps=eps, n_iters=n_iters, check_every=ce, ws=ws, f=f, g=g,
                                              trace=trace, check=False)),
            "cost": part_ms(lambda: sk.cost(A, B, f, g, eps=eps, out=cost_out)),
            "marginal_residual": part_ms(lambda: sk.marginal_residual(X, Y, A, B, f, g, eps=eps, ws=ws)),
        }
        if w.grad:
            parts["grad_x"] = part_ms(lambda: sk.grad_x(X, Y, A, B, g, eps=eps, ws=ws, out=grad))
        extra = {"components_ms": {k: round(v, 4) for k, v in parts.items()},
                 "solve_pair_evals_per_s": 2.0 * n * m * n_iters / (parts["solve"] * 1e-3),
                 "solve_iters_per_s": n_iters / (parts["solve"] * 1e-3)}
    if mode in ("marginal", "potential"):
        # the same iterations without checks, with the same pass timing events
        # as the timed steps: what the stop rule costs on top
        sk.solve_ex(X, Y, A, B, eps=eps, max_iter=counted_iters, ws=ws, f=f, g=g, check=False)
        torch.cuda.synchronize()
        sk.timing_enable(not args.graph, args.timing_stride)
        t2 = time.perf_counter()
        for _ in range(args.steps):
            sk.solve_ex(X, Y, A, B, eps=eps, max_iter=counted_iters, ws=ws, f=f, g=g, check=False)
        torch.cuda.synchronize()
        fixed_s = (time.perf_counter() - t2) / args.steps
        sk.timing_enable(False)
        extra = {"stop_mode": mode, "stop_tol": args.stop_tol, "check_every": args.check_every,
                 "iters_run": counted_iters, "converged": stop["converged"], "final_viol": stop["final_viol"],
                 "fixed_run_ms": fixed_s * 1e3, "stop_rule_overhead": step_s / fixed_s - 1.0}
    elif mode == "symmetric":
        extra = {"variant": "symmetric", "alpha": args.alpha}
    elif mode == "divergence":
        extra = {"divergence": [float(v) for v in dv_out.cpu()]}
    elif mode == "fs2":
        # the all-particle residual takes two dense passes: skipped beyond about an hour's reach of them
        dense_ok = float(n) * float(m) <= 2.0e14
        r = sk.marginal_residual(X, Y, A, B, f, g, eps=eps) if dense_ok else None
        # the order, blocks, coarse stage and lift alone (no fine iteration, so no screening), outside the timing
        torch.cuda.synchronize()
        t4 = time.perf_counter()
        sk.fs2_solve(X, Y, A, B, eps=eps, block=args.fs2_block, tol=fs2_tol, delta=args.fs2_delta, max_iters=0,
                     ws=ws_fs2, check=False)
        torch.cuda.synchronize()
        coarse_s = time.perf_counter() - t4
        extra = {"fs2": {k: v for k, v in fs2_info.items() if not k.startswith("perm")}, "fs2_tol": fs2_tol,
                 "coarse_stage_s": coarse_s,
                 "block": args.fs2_block, "delta": args.fs2_delta, "solve_s": step_s, "workspace_mb": nb / 1e6,
                 "all_particle_residual": float(max(r[0].item(), r[1].item())) if dense_ok else None}
        if args.fs2_dense:
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            _, _, it_d, conv_d, viol_d = sk.solve_ex(X, Y, A, B, eps=eps, stop_mode="marginal", stop_tol=fs2_tol,
                                                     max_iter=args.fs2_max_iters, check_every=10, ws=ws, check=False)
            torch.cuda.synchronize()
            extra["dense"] = {"solve_s": time.perf_counter() - t3, "iters": it_d, "converged": conv_d,
                              "final_viol": viol_d}
    elif mode == "hvp":
        extra = {"cg_iters": args.cg_iters, "cg_resid": float(cg_res.item()), "hvp_per_s": 1.0 / step_s}
    elif mode == "flow":
        extra = {"lr": args.lr, "flow_steps_per_s": 1.0 / step_s,
                 "flow_steps_run": args.warmup + args.steps + (1 if args.graph else 0) * 2}
    value = pair_evals / step_s
    avg_launch_s = pass_ms * 1e-3 / launches if launches else float("nan")
    pairs_per_launch = pairs / launches if launches else float("nan")
    if mode == "primal":
        roof = None  # two kinds of pass per call (a weighted transport pass and a column pass): timed as a whole
    elif mode == "fs2":
        # the block-sparse pass over the kept tiles: the dense pass's per-pair work
        roof = roofline_alu(d, pairs_per_launch, avg_launch_s) if launches else None
        if roof is not None:
            roof["kernel"] = f"k_pass_sparse<{d}>"
    elif mode == "grad":
        if d > 8:
            # transport mode 4: split scores, then the key coordinates as a P-column payload (the weighted sums
            # in the fp16 split form up to a padded width of 128, fp32 beyond)
            roof = roofline_transport_split(d, pairs_per_launch, avg_launch_s, d, cols=packed_stride(d),
                                            split_sums=packed_stride(d) <= 128)
            roof["kernel"] = "k_transport_mfma<%d,1,4>" % packed_stride(d)
        else:
            roof = None  # the vector-ALU gradient is timed as a part of the default solve step (components_ms)
    elif mode in ("hvp", "transport"):
        payload = 1 if mode == "hvp" else d  # columns of the dominant launches (CG steps / the product)
        if d > 8 and payload > 1:
            payload = min(payload, 64 if packed_stride(d) >= 64 else 16)  # one launch's chunk of columns
        if d <= 8:
            roof = roofline_alu(d, pairs_per_launch, avg_launch_s, payload)
            roof["kernel"] = "k_transport<%d,%d,0>" % (d, 1 if payload == 1 else (4 if payload <= 4 else 9))
        else:
            p2 = packed_stride(d)
            if payload == 1:
                # the one-column kernel forms its scores in the split form (payload FMAs on the vector ALUs)
                roof = roofline_split(d, pairs_per_launch, avg_launch_s)
            else:
                # the payload's weighted sums in the fp16 split form up to a padded width of 128
                roof = roofline_transport_split(d, pairs_per_launch, avg_launch_s, payload, split_sums=p2 <= 128)
            # one column: MODE 3 (vector-ALU payload); d columns: 16- or 64-column tiles (MODE 0)
            roof["kernel"] = ("k_transport_mfma<%d,1,3>" % p2 if payload == 1 else
                              "k_transport_mfma<%d,%d,0>" % (p2, 4 if payload > 16 else 1))
    elif d <= 8:
        roof = roofline_alu(d, pairs_per_launch, avg_launch_s)
        small = pairs_per_launch <= 2.0e6  # the library's single-kernel path for small passes
        roof["kernel"] = f"k_pass_small<{d}>" if small else f"k_pass_valu<{d}>"
    else:
        roof = roofline_split(d, pairs_per_launch, avg_launch_s)
        roof["kernel"] = "k_pass_mfma<%d>" % packed_stride(d)
    if roof is not None and mode != "fs2" and args.size is None and args.dim is None:
        # the counter runs were taken on the workload at its own shape
        roof["traffic"] = load_traffic(f"{args.workload}:pass", "valu" if d <= 8 else "mfma", roof["kernel"])
    elif roof is not None and mode != "fs2":
        roof["traffic"] = None
    elif roof is not None:
        roof["traffic"] = None  # no counter run of the sparse pass

    out = {
        "metric": "point-pair evals/sec and Sinkhorn iters/sec (n=m=50k,d=3); % fp32 peak",
        "value": value,
        "unit": "pair-evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload + ("" if args.dim is None else " (d = %d)" % d), "n": n, "m": m,
                   "d": d, "eps": eps,
                   # the two-stage solver runs to its target or its iteration cap, without the gradient
                   "n_iters": args.fs2_max_iters if mode == "fs2" else n_iters,
                   "check_every": ce if mode != "fs2" else 10, "grad_x": bool(w.grad) and mode != "fs2",
                   "eps_rule": "n^(-2/3) at n = %d" % n if args.eps_blur else "the workload's",
                   "recipe": w.description},
        "mode": mode,
        "iters_per_s": (3 * n_iters if mode == "divergence" else
                        fs2_info["fine_iters"] if mode == "fs2" else counted_iters) / step_s,
        "hip_graph": bool(args.graph),
        "pass_pair_evals_per_s": pairs_per_launch / avg_launch_s if (launches and mode != "primal") else None,
        "roofline": roof,
        "final_residual": float(trace[n_iters // ce - 1].item()) if (ce and mode == "solve") else None,
        "cost": (float(cost_out.item()) if mode not in ("divergence", "hvp", "transport", "fs2", "primal") else
                 float(primal_out[0].item()) if mode == "primal" else None),
        **extra,
    }
    if not args.no_cpu_baseline and mode == "solve":
        out["cpu_baseline"] = cpu_baseline(x, y, a, b, eps, n, m)
    if mode == "solve" and not args.graph and args.workload == "gmm8_d3_sq" and args.size is None \
            and args.dim is None and args.iters is None and not args.no_extra_configs:
        del X, Y, A, B, ws, f, g, grad
        torch.cuda.empty_cache()
        configs = []
        for name, steps, use_graph, iters in EXTRA_CONFIGS:
            configs.append(run_extra_config(name, steps, use_graph, iters, args.timing_stride))
            print(f"extra config done: {name}", file=sys.stderr, flush=True)
        out["extra"] = {"configs": configs}
    print(json.dumps(out), flush=True)


# The other workloads, timed after the headline by the default run: (name, timed steps, HIP-graph replay,
# iterations per step or None for the workload's own count).  The 2^20-point workload is timed on 2 of its
# 50 iterations and the cost, without its gradient (a full step takes about 19 s); its entry says so.
EXTRA_CONFIGS = [("gflow_d2", 20, True, None), ("gauss_d2", 5, True, None), ("gmm8_d3", 3, False, None),
                 ("gauss_d64", 3, True, None), ("cluster_d3", 1, False, 2)]


def run_extra_config(name: str, steps: int, graph: bool, iters, timing_stride: int) -> dict:
    """One workload's step, as the default mode runs it (sk_solve with the workload's residual interval, sk_cost,
    sk_grad_x when the workload has one), with one warm-up step; returns its line for extra.configs."""
    import torch

    import streaming_sinkhorn_solver_amd as sk
    from sk_inputs import WORKLOADS, eps32, make_inputs

    w = WORKLOADS[name]
    n_iters = w.n_iters if iters is None else iters
    eps = eps32(w.eps)
    x, y, a, b = make_inputs(name)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    dev = torch.device("cuda:0")
    X, Y, A, B = (torch.from_numpy(v).to(dev) for v in (x, y, a, b))
    ws = sk.workspace(n, m, d, dev)
    f = torch.empty(n, dtype=torch.float32, device=dev)
    g = torch.empty(m, dtype=torch.float32, device=dev)
    ce = w.check_every if n_iters >= max(w.check_every, 1) else 0
    trace = torch.empty(max(n_iters // ce, 1) if ce else 1, dtype=torch.float32, device=dev)
    cost_out = torch.empty(1, dtype=torch.float64, device=dev)
    grad = torch.empty((n, d), dtype=torch.float32, device=dev)
    sk.check_inputs(X, Y, A, B, ws)

    with_grad = w.grad and iters is None  # a step cut to a few iterations times the iterations alone

    def step():
        sk.solve(X, Y, A, B, eps=eps, n_iters=n_iters, check_every=ce, ws=ws, f=f, g=g, trace=trace, check=False)
        sk.cost(A, B, f, g, eps=eps, out=cost_out)
        if with_grad:
            sk.grad_x(X, Y, A, B, g, eps=eps, ws=ws, out=grad)

    step()
    torch.cuda.synchronize()
    sk.timing_enable(True, timing_stride)
    cuda_graph = None
    if graph:  # kernel durations from one eager step; the timed steps replay the graph
        step()
        torch.cuda.synchronize()
        pass_ms, launches, pairs = sk.timing_read()
        sk.timing_enable(False)
        cuda_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cuda_graph):
            step()
        cuda_graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        cuda_graph.replay() if cuda_graph is not None else step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    if cuda_graph is None:
        pass_ms, launches, pairs = sk.timing_read()
        sk.timing_enable(False)
    avg_s = pass_ms * 1e-3 / launches
    ppl = pairs / launches
    if d <= 8:
        roof = roofline_alu(d, ppl, avg_s)
        roof["kernel"] = f"k_pass_small<{d}>" if ppl <= 2.0e6 else f"k_pass_valu<{d}>"
        roof["traffic"] = load_traffic(f"{name}:pass", "valu", roof["kernel"])
    else:
        roof = roofline_split(d, ppl, avg_s)
        roof["kernel"] = "k_pass_mfma<%d>" % packed_stride(d)
        roof["traffic"] = load_traffic(f"{name}:pass", "mfma", roof["kernel"])
    out = {"workload": name, "n": n, "m": m, "d": d, "eps": eps, "n_iters": n_iters, "check_every": ce,
           "grad_x": bool(with_grad), "steps": steps, "hip_graph": graph, "ms_per_step": step_s * 1e3,
           "value": 2.0 * n * m * n_iters / step_s, "unit": "pair-evals/s", "iters_per_s": n_iters / step_s,
           "roofline": roof, "recipe": w.description}
    if iters is not None:
        out["note"] = (f"{n_iters} of the workload's {w.n_iters} iterations per timed step, with the cost and "
                       f"without the gradient")
    del X, Y, A, B, ws, f, g, grad
    torch.cuda.empty_cache()
    return out


def cpu_baseline(x, y, a, b, eps, n, m) -> dict:
    """The CPU oracle as it stands, on a bounded sample of the same problem: alternating iterations from
    g = 0, as many as fill about 10 s of wall time (one timed iteration sets the count, at most 30 s)."""
    import math

    import oracle

    lib = oracle.load()
    t0 = time.perf_counter()
    oracle.sinkhorn(x, y, a, b, eps, 1, lib=lib)
    t1 = time.perf_counter() - t0
    k = max(1, min(math.ceil(10.0 / t1), math.floor(30.0 / t1)))
    t0 = time.perf_counter()
    oracle.sinkhorn(x, y, a, b, eps, k, lib=lib)
    dt = time.perf_counter() - t0
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": 2.0 * n * m * k / dt, "unit": "pair-evals/s", "cores": oracle.num_threads(lib), "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"{k} full alternating iterations (row + column half-steps, {2 * n * m * k:.3g} pair evaluations) "
                      f"of the same workload from g = 0, float64, {dt:.1f} s wall (after one timed iteration "
                      f"that sets the count)"}


if __name__ == "__main__":
    main()
