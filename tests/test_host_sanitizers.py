"""The library's host code (C entry points and their validation, the slot
cache's policy and bookkeeping, the tensor-parallel slicer's checks) under
AddressSanitizer and UndefinedBehaviorSanitizer: the CPU suites that drive
it through the C ABI run again, in a child process that preloads the ASan
runtime, against a build whose host objects are instrumented.  Any sanitizer
report fails the run (UBSan is built without recovery, ASan halts on error).
No GPU: every call these suites make either runs on the host or fails its
validation before anything is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SUITES = ["tests/test_cache_host.py", "tests/test_abi.py"]


def test_host_code_under_asan_and_ubsan():
    from mxfp4_routed_expert_renorm_amd import build as B
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": B.asan_runtime(),
        # Python and its extension modules are not instrumented: leak reports
        # and ODR checks would be about them, not about the library
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "MOE_TEST_LIBRARY": lib,
    })
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-p", "no:xdist", *SUITES]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = p.stdout + p.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
