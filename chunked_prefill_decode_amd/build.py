"""Compile libsarathi_attn.so in-tree for gfx950 with hipcc.

build()                 -- the library itself;
build(sanitize=True)    -- libsarathi_attn_san.so: the same sources with
                           AddressSanitizer and UndefinedBehaviorSanitizer on
                           the host code only (the device code is unchanged);
                           for running the host-side tests on the CPU
                           (tests/test_host_sanitized.py).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/sched.cpp", "csrc/plan.cpp", "csrc/misc.cpp", "csrc/kernels.hip", "csrc/linear.hip"]
OUT = os.path.join(HERE, "libsarathi_attn.so")
OUT_SAN = os.path.join(HERE, "libsarathi_attn_san.so")
# Packed fp32 instructions are kept out of the device code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         # the kernels never produce NaN (masked scores are selected to -inf, cache
         # slots past a sequence are zeroed), so max() needs no NaN canonicalisation
         "-fno-honor-nans"]
# Host-side sanitizers (each flag bound to the host compilation).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libsan", "-g"]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized library needs preloaded."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = OUT_SAN if sanitize else OUT
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *(SAN_FLAGS if sanitize else []), "-I" + os.path.join(ROOT, "include")]
    cmd += [os.path.join(HERE, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
