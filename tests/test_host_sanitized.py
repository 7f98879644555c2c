"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: a build with sanitized host code (the device code as usual) runs
the CPU tests of the argument checks, the configuration choice, the tuner's
candidates and cache parser, the host-resident planner, the binding's checks
and the C99 program, in a child process with the sanitizer runtime preloaded.
Any report (an out-of-bounds access, a use after free, undefined behaviour)
ends that process with an error."""
import os
import subprocess
import sys

import pytest

from fp32_gemm_02_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitized")
INNER = ["tests/test_host_plan.py", "tests/test_tune_cache.py", "tests/test_c_abi.py",
         "tests/test_abi.py", "tests/test_binding_checks.py"]


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = hip_build.SOURCES + [os.path.join(ROOT, "include", "phobos_sgemm.h")] + [
        os.path.join(hip_build.HERE, "csrc", f) for f in os.listdir(os.path.join(hip_build.HERE, "csrc"))]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.mark.timeout(900)
def test_host_code_is_clean_under_sanitizers():
    rt = hip_build.asan_runtime()
    if rt is None:
        pytest.skip("no shared AddressSanitizer runtime next to the compiler")
    lib = os.path.join(OUT, "libphobos_sgemm.so")
    if _stale(lib):
        hip_build.build_sanitized(OUT)
    env = dict(os.environ, LD_PRELOAD=rt, PHOBOS_SGEMM_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *INNER, "-m", "not gpu", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=800)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
