"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer. Builds libhga_hostsan.so (the library with its
host-side argument checks, workspace sizing and dispatch instrumented; device
code untouched) and runs the ABI tests against it in a child process with the
compiler's ASan runtime preloaded. Those tests exercise every validation and
error path without launching GPU work, so they run here without a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = ("import sys\n"
          "import long_context_fine_amd.hga as h\n"
          "h._LIB_PATH = sys.argv[1]\n"
          "import pytest\n"
          "sys.exit(pytest.main([sys.argv[2], '-q', '-m', 'not gpu', '-p', 'no:cacheprovider']))\n")


def test_abi_checks_are_clean_under_asan_and_ubsan():
    from long_context_fine_amd import build
    try:
        lib = build.build_host_sanitized()
        runtime = build.asan_runtime()
    except RuntimeError as e:  # no ROCm compiler with sanitizer runtimes here
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", _CHILD, lib, os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout
