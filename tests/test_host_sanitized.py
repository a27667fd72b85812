"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host side is built with both sanitizers (no device code), and
the host ABI tests (argument validation that must write nothing, the policy
table, workspace sizes, status strings, kernel selection) run against it in a
child process with the sanitizer runtime preloaded. Any report fails the test.
"""

import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from mx_bit_quantized_amd import _build  # noqa: E402


def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    rt = _build.sanitizer_runtime()
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    lib = _build.build_host_sanitized(str(tmp_path / "libmxq_asan.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "MXQ_TEST_LIB": lib,
        # the interpreter and numpy are not instrumented: leaks and their
        # allocator pairs are theirs, not the library's
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                          "-p", "no:cacheprovider", "-k", "not refuses_cpu_tensors"],
                         cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = res.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
