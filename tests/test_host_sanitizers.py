"""The host-side tests (argument checks, the fold, the band constants, the no-alloc size limit)
against a build of libtri whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer:
an out-of-bounds access, a use after free or undefined behaviour in the host code fails the run.
Builds the library into a temporary directory (about half a minute) and runs the tests in a
child process with the ASan runtime preloaded."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_under_asan_and_ubsan(tmp_path):
    from rotary_frequency_key_amd import build as B

    try:
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized(str(tmp_path / "libtri_sanitized.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host code is instrumented
    env = dict(os.environ, TRI_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          "tests/test_abi_cpu.py", "tests/test_zz_no_alloc.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
