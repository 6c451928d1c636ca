"""Compile libsarathi_attn.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/sched.cpp", "csrc/plan.cpp", "csrc/misc.cpp", "csrc/kernels.hip", "csrc/linear.hip"]
OUT = os.path.join(HERE, "libsarathi_attn.so")
# Packed fp32 instructions are kept out of the device code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         # the kernels never produce NaN (masked scores are selected to -inf, cache
         # slots past a sequence are zeroed), so max() needs no NaN canonicalisation
         "-fno-honor-nans"]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc, *FLAGS, "-I" + os.path.join(ROOT, "include")] + [os.path.join(HERE, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
