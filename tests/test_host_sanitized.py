"""The host-side tests again, against the library built with AddressSanitizer
and UndefinedBehaviorSanitizer on its host code (batch builder, commit,
metadata packing, argument checks).  Any invalid memory access or undefined
behaviour aborts the child run, which fails this test.  No kernel runs here.

The sanitized library is built by __graft_entry__.build() (or
`python chunked_prefill_decode_amd/build.py --sanitize`)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "chunked_prefill_decode_amd", "libsarathi_attn_san.so")
HOST_TESTS = ["tests/test_native_sched.py", "tests/test_plan.py", "tests/test_policies.py", "tests/test_abi.py",
              "tests/test_linear_host.py", "tests/test_zz_no_alloc.py"]


@pytest.mark.timeout(600)
def test_host_tests_pass_under_asan_and_ubsan():
    if not os.path.exists(SAN_LIB):
        pytest.skip("sanitized library not built (python chunked_prefill_decode_amd/build.py --sanitize)")
    sys.path.insert(0, ROOT)
    from chunked_prefill_decode_amd.build import sanitizer_runtime
    env = dict(os.environ, SARATHI_ATTN_LIB=SAN_LIB, LD_PRELOAD=sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
                       + HOST_TESTS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=580)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
