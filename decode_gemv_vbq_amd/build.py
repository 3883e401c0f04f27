"""Build libvbq.so (gfx950) in-tree with hipcc.

    python -m decode_gemv_vbq_amd.build            # build
    python -m decode_gemv_vbq_amd.build --asm DIR  # also keep the AMD ISA of the kernels
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvbq.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def command(out: str, extra=()):
    return (["hipcc", "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
             "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS + list(extra) + ["-o", out] + sources())


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    extra = []
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        extra = ["-save-temps"]
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = asm_dir or None
    if asm_dir:
        # -save-temps writes the intermediates into the working directory
        cmd = [c for c in cmd]
    subprocess.check_call(cmd, cwd=cwd)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (AMD ISA) in this directory")
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.asm, a.v))


if __name__ == "__main__":
    sys.exit(main())
