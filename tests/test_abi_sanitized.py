"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer.

fp4_api.cpp (every validation path of the boundary) is built as host C++
with both sanitizers, every UB report fatal, and linked with stand-ins for
the kernel launchers (build.py build_sanitized).  tests/test_abi.py then runs
against that library in a child process with the sanitizer runtime
preloaded; any out-of-bounds access, use of freed memory or undefined
behaviour aborts it.  (This found one: C++ leaves loading an out-of-range
value into an enum without a fixed underlying type undefined, which the
checks of bad enum arguments did; the headers now fix every enum to int.)
"""
import os
import subprocess
import sys

import pytest

from fp4_block_scaled_x16_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(build.CLANG), reason="clang++ of ROCm not installed")
def test_abi_checks_under_asan_and_ubsan():
    lib = build.build_sanitized()
    runtime = build.sanitizer_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, FP4_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = p.stdout[-3000:] + p.stderr[-3000:]
    assert p.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert " passed" in p.stdout
