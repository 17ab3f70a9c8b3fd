"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The step builder (cb_sched_*), the launch planner (cb_plan_describe), argument checks and
the entry points' host paths are rebuilt with host-side sanitizers (device code unchanged;
build.py --sanitize) and the CPU tests that drive them - bit-exact scheduler parity against
the Python reference over long traces with arrivals, EOS, preemption and naive batching,
the planner's rules, and every ABI argument check - run again in a child process that
preloads the clang ASan runtime and loads that copy. Any heap or stack overflow,
use-after-free, or undefined behaviour (signed overflow, misaligned or null access, bad
shift) aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

from ragged_continuous_batching_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_sched_parity.py", "tests/test_plan.py", "tests/test_abi.py"]


def sanitized_env(lib):
    return dict(os.environ, LD_PRELOAD=B.asan_runtime(), CB_LIBRARY=lib,
                ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        lib = B.build(jobs=min(8, os.cpu_count() or 1), sanitize=True)
    except (RuntimeError, FileNotFoundError) as e:       # pragma: no cover (no hipcc)
        pytest.skip(f"sanitized build unavailable: {e}")
    with open(lib, "rb") as f:
        assert b"__asan_report_load" in f.read(), "the test copy carries no ASan checks"
    return lib


def test_sanitized_copy_is_the_one_loaded(sanitized_lib):
    code = ("from ragged_continuous_batching_amd import cb; import sys; "
            "maps = open('/proc/self/maps').read(); "
            "sys.exit(0 if cb.LIB_PATH in maps and 'libclang_rt.asan' in maps else 3)")
    r = subprocess.run([sys.executable, "-c", code], env=sanitized_env(sanitized_lib), cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_host_code_under_asan_and_ubsan(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", *SUITES, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       env=sanitized_env(sanitized_lib), cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
