"""The CPU tests that load the library, rerun against a host build instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer.

tri_mul.cpp, pair_transition.cpp and tri_attention.cpp (argument checks, plans, weight
folding and every LDS image builder) are compiled host-only with both sanitizers and
linked with the plain kernel objects into _build_san/libtrimul_san.so; a child pytest
with the sanitizer runtime preloaded then runs tests/test_abi_cpu.py and
tests/test_host_images.py against it. Any ASan report aborts the child, any UBSan report
is fatal, and either fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

from pair_rep_triangle_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _toolchain():
    if not os.path.exists(B.HIPCC) or shutil.which("nm") is None:
        return None
    return B.sanitizer_runtime()


@pytest.mark.timeout(900)
def test_library_host_code_is_clean_under_asan_and_ubsan():
    runtime = _toolchain()
    if runtime is None:
        pytest.skip("hipcc, nm or the compiler's ASan runtime is not available")
    lib = B.build_sanitized(verbose=False)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "library not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["PAIR_REP_TRIANGLE_LIB"] = lib
    # Python itself is not instrumented and keeps its allocations to the end: no leak check
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:check_initialization_order=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_host_images.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
