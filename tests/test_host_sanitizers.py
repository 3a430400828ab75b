"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer.

The build makes a second copy of the library whose host code (argument
validation, schedules, the recompute-ratio controller, the LRU replay, plan
sizing) is instrumented; its GPU code is the same.  This test runs the CPU
ABI tests against that copy in a child process with the ASan runtime
preloaded and fails on any sanitizer report.  No kernel is launched."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "non_prefix_kv_amd", "_build_san", "libcacheblend_san.so")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_tests_clean_under_asan_ubsan():
    rt = _asan_runtime()
    if not os.path.exists(SAN_LIB) or rt is None:
        pytest.skip("sanitized library or ASan runtime not present")
    nm = subprocess.run(["nm", "-D", "--undefined-only", SAN_LIB], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout and "__ubsan_handle_" in nm.stdout, \
        "the sanitized library carries no instrumentation"
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, CACHEBLEND_LIB=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import non_prefix_kv_amd as n; "
             "print(any('libcacheblend_san.so' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("True"), r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join("tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
