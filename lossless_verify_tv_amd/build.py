"""Build ``liblvtv.so`` (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m lossless_verify_tv_amd.build`` (or ``build()`` from
Python). The library lands next to this file; the Python binding loads it
from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblvtv.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "verify_rows.hip", "loss.hip", "loss_fused.hip", "schedule.hip"]

# -ffp-contract=off: products that must round on their own (the canonical
# scaled logit) are never fused; kernels request fused multiply-adds
# explicitly. Packed fp32 instructions are disabled for all HIP code.
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblvtv.so)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblvtv.so; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    if verbose and res.stderr.strip():
        print(res.stderr[-3000:], file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
