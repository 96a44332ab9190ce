"""Build librs.so (the gfx950 HIP library behind include/rs.h) in-tree.

    python -m lsd_radix_sort_pass_amd.build [--save-temps DIR]

Always recompiles.  The library is written to lsd_radix_sort_pass_amd/librs.so.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librs.so")
SOURCES = [os.path.join(CSRC, "rs.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed FP32 instructions are kept out of every code object.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", out_tmp, *SOURCES]
    cwd = PKG
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps")
        cwd = save_temps
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(out_tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) in this directory")
    args = ap.parse_args(argv)
    path = build(args.save_temps, verbose=True)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
