"""Builds the HIP shared library libsk.so for gfx950, in-tree.

Usage: ``python -m streaming_sinkhorn_solver_amd.build`` (or call ``build()``).
Every HIP source under csrc/ is compiled by one hipcc invocation into
``streaming_sinkhorn_solver_amd/_build/libsk.so``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libsk.so")
UBENCH_PATH = os.path.join(BUILD_DIR, "libsk_ubench.so")
ARCH = "gfx950"

# Packed-fp32 VALU instructions are disabled for the device code: the compiler
# must emit scalar v_fma/v_add/v_mul_f32 only.  Matrix-core accumulators are
# kept in ordinary VGPRs (no AGPR copies before the LSE epilogue reads them).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def compile_command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
             "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS + (extra or [])
            + sources() + ["-o", out])


def _compile(cmd_for, out: str, verbose: bool) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = cmd_for(tmp)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (proc.returncode, " ".join(cmd), proc.stderr[-8000:]))
    if verbose:
        err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def ubench_command(out: str = UBENCH_PATH) -> list[str]:
    src = os.path.join(CSRC, "ubench", "sk_ubench.hip")
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared"] + DEVICE_FLAGS + [src,
                                                                                                        "-o", out]


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB_PATH) -> str:
    """Compile libsk.so and the issue-rate micro-benchmark library (always recompiles)."""
    _compile(lambda tmp: compile_command(tmp, extra), out, verbose)
    if out == LIB_PATH:
        _compile(ubench_command, UBENCH_PATH, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
