"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the host code of gqa_api.hip is built instrumented (device code
unchanged) and every check of test_abi.py runs against that build in a
child process with the sanitizer runtime preloaded.  A report of either
sanitizer fails the test.  (This run found that the status and dtype enums
could not hold every int a C caller may pass; they now have int as their
fixed underlying type in C++.)"""

import os
import subprocess
import sys

from grouped_query_attention_fwd_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_and_ubsan():
    lib = _build.build_sanitized()
    env = dict(os.environ,
               GQA_TEST_LIBRARY=lib,
               LD_PRELOAD=_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out
