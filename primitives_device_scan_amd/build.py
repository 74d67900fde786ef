"""Builds libdevscan.so (the HIP library behind include/devscan.h) in-tree.

    python primitives_device_scan_amd/build.py

(Run it as a script, not with -m: importing the package loads the library.)

Compiles every HIP source for gfx950 with hipcc. Packed fp32 instructions are
disabled for the device code (-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdevscan.so")
SOURCES = ["scan_lookback.hip", "scan_blocked.hip", "scan_three_pass.hip", "compact.hip", "compact_unordered.hip", "counting_sort.hip", "copy.hip", "tile_lds.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_flags(extra=()):
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra]


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    objs, procs = [], []
    for src in SOURCES:  # compile the sources in parallel
        obj = os.path.join(CSRC, src + ".o")
        cmd = [HIPCC, *hipcc_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        objs.append(obj)
    for cmd, p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
