"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: capi.cpp and plan.cpp built by g++ with host-only
stand-ins for the kernel launchers (tests/capi_host/), then a seeded fuzz
over every entry point.  No GPU is involved: the stand-ins launch nothing.

The fuzz asserts that every call returns a status of the header's set, that
a refused call launched nothing, and that a workspace of the size the
matching size query returned is never refused; the sanitizers abort on any
overrun (this is how a rotary table larger than the library's 128-pair
buffer once wrote past it) or signed overflow in the range checks."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "capi_host"))


@pytest.fixture(scope="module")
def fuzz_exe():
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    import build as capi_host_build
    return capi_host_build.build()


@pytest.mark.parametrize("seed", [1, 20251202])
def test_sanitized_fuzz_of_every_entry_point(fuzz_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe, "40000", str(seed)], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
    accepted = int(r.stdout.split(" accepted calls")[0].rsplit(" ", 1)[1])
    assert accepted > 1000, r.stdout      # the fuzz reaches the launches, not only the checks
