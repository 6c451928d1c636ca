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
