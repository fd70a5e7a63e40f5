"""The host code of the C ABI (argument validation, planning, launch
sequencing) under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is rebuilt with both on its host code only, and the CPU validation
tests of tests/test_abi.py run against that build in a child process with
the sanitizer runtime preloaded.  Any report fails the test (CPU only)."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    for pat in ("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def test_abi_validation_under_asan_and_ubsan():
    from kv_cache_rate_amd import build
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm installation")
    lib = build.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ)
    env.update(KVQ_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
