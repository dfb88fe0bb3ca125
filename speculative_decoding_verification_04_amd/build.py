"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_decoding_verification_04_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libspecverify.so")
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def command(out: str = LIB) -> list:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            # packed fp32 instructions stay off on this target
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
            *srcs, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


BENCH_FLOOR_SRC = os.path.join(ROOT, "bench_floor.hip")
BENCH_FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")


def build_bench_floor(verbose: bool = False) -> str:
    """Compile bench.py's read-floor probe (a measurement aid beside bench.py,
    not part of the library) into bench_floor.so at the repository root."""
    tmp = BENCH_FLOOR_LIB + ".tmp"
    cmd = [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-command-line-argument", BENCH_FLOOR_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    os.replace(tmp, BENCH_FLOOR_LIB)
    return BENCH_FLOOR_LIB


if __name__ == "__main__":
    print(build(verbose=True))
