"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with both sanitizers on its host code (build_sanitized.py; the device
code is unchanged), and the CPU tests of the ABI (tests/test_abi.py: symbol exports, every
validation path, workspace sizes, the capacity helper) run against it in a child process with
the sanitizer runtime preloaded and every report fatal. A memory error or undefined behaviour in
argument checking, layout arithmetic or the helpers fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    from sparse_mixture_experts_02_amd import build_sanitized as build
    rt = build.sanitizer_runtime()
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm installation")
    lib = build.build_host_sanitized()
    # the library really is instrumented (it calls the sanitizer runtime)
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_" in nm.stdout and "__ubsan_handle_" in nm.stdout
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + env.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", MOE_TEST_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
