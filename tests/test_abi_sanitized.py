"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

The library's host code (validation, launch planning, workspace layout) is
its error path: every bad argument must be refused there before any HIP
call.  This builds the library with ASan + UBSan on the host code
(``long_context_verify_amd.build.build_sanitized``) and runs the host-check
tests of ``test_abi_cpu.py`` against it in a child process with the sanitizer
runtime preloaded; any sanitizer report fails the test.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources_newer_than(lib):
    from long_context_verify_amd import build as B
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(B.CSRC, s) for s in os.listdir(B.CSRC)] + [
        os.path.join(B.INCLUDE, h) for h in os.listdir(B.INCLUDE)]
    return any(os.path.getmtime(s) > t for s in srcs)


def test_host_checks_are_clean_under_asan_and_ubsan():
    from long_context_verify_amd import build as B
    lib = B.SANITIZED_LIB_PATH
    if _sources_newer_than(lib):
        B.build_sanitized()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "library is not instrumented"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": B.sanitizer_runtime(),
        "SPECVERIFY_LIB": lib,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-k", "not bench_refuses"],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
