"""The shared library loads on the CPU and exports every entry point that
include/sarathi_attn.h declares (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_api():
    names = declared_functions()
    for n in ["sa_build_batch", "sa_kv_append", "sa_hybrid_attn", "sa_sched_commit", "sa_batch_upload"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    from chunked_prefill_decode_amd import native as N
    lib = ctypes.CDLL(N.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) <= set(N.EXPORTED)


def test_version_and_error_text():
    from chunked_prefill_decode_amd import native as N
    assert "gfx950" in N.sa_version()
    with pytest.raises(N.SarathiError) as e:
        N.sa_sched_create(8, 4, [0, 0])
    assert "permutation" in e.value.message


def test_library_shares_torchs_hip_runtime():
    """Importing the binding before anything else has loaded torch, and torch
    after it, leaves one HIP runtime and one HSA runtime in the process: the
    library binds to the one torch holds, never to a second copy, whose calls
    would find no device."""
    import subprocess
    import sys
    code = ("import chunked_prefill_decode_amd.native\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if '/' in l}\n"
            "print(sum('libamdhip64' in m for m in maps), sum('libhsa-runtime64' in m for m in maps))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[-2:] == ["1", "1"], r.stdout
