"""Build libqopt.so (HIP for gfx950 + host C++) in-tree with hipcc.

    python block_wise_bit_adam8bit_amd/build.py [--save-temps]

(run by path: importing the package would open the library this script builds)

Flags that matter for results: -ffp-contract=off (no fused multiply-add, so every
binary32 operation rounds once, as the update is defined); no fast-math (IEEE
divide and square root, fp32 denormals kept); packed fp32 ops disabled.
"""

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqopt.so")

ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra",
          "-Wno-unused-parameter", "-I", INCLUDE]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _hipcc():
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found ({cand})")
    return cand


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}")
    return res.stdout


def build(verbose=False, save_temps=False, extra_defines=()):
    """Compile every source and link libqopt.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    defs = [f"-D{d}" for d in extra_defines]
    host_obj = os.path.join(BUILD, "codebook.o")
    _run([hipcc, "-x", "c++", *COMMON, *defs, "-c", os.path.join(CSRC, "codebook.cpp"),
          "-o", host_obj], verbose)
    temps = ["-save-temps=obj"] if save_temps else []
    dev_objs = []
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        obj = os.path.join(BUILD, src[:-4] + ".o")
        _run([hipcc, "-x", "hip", *COMMON, *DEVICE, *defs, *temps, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        dev_objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", host_obj, *dev_objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-q", "--quiet", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=not args.quiet, save_temps=args.save_temps)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
