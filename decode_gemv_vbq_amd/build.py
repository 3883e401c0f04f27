"""Build libvbq.so (gfx950) in-tree with hipcc.

    python -m decode_gemv_vbq_amd.build            # build
    python -m decode_gemv_vbq_amd.build --asm DIR  # also keep the AMD ISA of the kernels
"""
from __future__ import annotations

import argparse
import concurrent.futures
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

# Per-source device flags.  vbq_plan.hip: the one-matrix decode kernel takes its
# record as 13 scalar arguments, which the dispatch preloads into SGPRs (gfx950
# kernel-argument preloading), so no wavefront waits on a load of its arguments.
SOURCE_FLAGS = {"vbq_plan.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=13"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


OBJDIR = os.path.join(ROOT, "_build")


def compile_command(src: str, obj: str, extra=()):
    return (["hipcc", "-O3", "-std=c++17", "-fPIC", "-c", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
             "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS + list(extra) + ["-o", obj, src])


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libvbq.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    extra = []
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        extra = ["-save-temps"]  # writes the intermediates into the working directory
    jobs = []
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
        jobs.append((compile_command(src, obj, SOURCE_FLAGS.get(os.path.basename(src), []) + extra), obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = []
        for cmd, _ in jobs:
            if verbose:
                print(" ".join(cmd), flush=True)
            futs.append(ex.submit(subprocess.run, cmd, cwd=asm_dir or None, capture_output=True, text=True))
        failed = []
        for (cmd, _), f in zip(jobs, futs):
            r = f.result()
            if r.returncode != 0:
                failed.append(r.stderr)
            elif verbose and r.stderr:
                print(r.stderr, file=sys.stderr)
    if failed:
        sys.stderr.write("\n".join(failed))
        raise subprocess.CalledProcessError(1, "hipcc")
    tmp = LIB + ".tmp"
    link = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in jobs]
    subprocess.check_call(link)
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
