"""The library's host code (argument validation, workspace arithmetic, last-call state)
under AddressSanitizer and UndefinedBehaviorSanitizer: libpnr_san.so is built on demand
(the device code is compiled as usual; only the host passes are instrumented) and
tests/host_sanitized_driver.py runs against it in a child process with the sanitizer
runtime preloaded.  No device call is made: this runs on the CPU.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "nonlinear_rnn_evaluation_amd")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(s) > t for s in glob.glob(os.path.join(PKG, "csrc", "*")) +
               [os.path.join(ROOT, "include", "pnr.h")])


@pytest.mark.skipif(_asan_runtime() is None, reason="no AddressSanitizer runtime in this toolchain")
def test_host_code_under_address_and_undefined_behavior_sanitizers():
    sys.path.insert(0, ROOT)
    from nonlinear_rnn_evaluation_amd.build import LIB_SANITIZED, build_library
    if _stale(LIB_SANITIZED):
        build_library(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_sanitized_driver.py"), LIB_SANITIZED],
                         env=env, capture_output=True, text=True, timeout=600)
    report = out.stdout + out.stderr
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert out.returncode == 0 and "host checks passed" in out.stdout, report[-4000:]
