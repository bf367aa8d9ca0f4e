"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Each test builds the sanitized variant (tests/sanitized_build.py, cached in
_build_san/) and runs CPU test files against it in a child process with the
matching ASan runtime preloaded: the oracle's pins under gcc's runtime, the
C ABI's host-side tests (argument validation, error paths, exports, the
grouping planner) under clang's.  Any sanitizer report fails the child
(UBSan does not recover), and so the test.
"""
import os
import subprocess
import sys

import pytest

import sanitized_build

ROOT = sanitized_build.ROOT
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _run_child(tests, extra_env):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra_env)
    # -s: a sanitizer report goes to the child's stderr, not into a capture the
    # halted child never prints
    cmd = [sys.executable, "-m", "pytest", *tests, "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


def test_oracle_under_sanitizers():
    try:
        lib = sanitized_build.build_oracle()
        runtime = sanitized_build.gcc_asan_runtime()
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    tests = ["tests/test_oracle_pins.py", "tests/test_oracle_properties.py", "tests/test_oracle_strided.py",
             "tests/test_oracle_grouping.py", "tests/test_box_map.py"]
    out = _run_child(tests, {"LD_PRELOAD": runtime, "SPCONV_ORACLE_LIB": lib})
    assert " passed" in out


def test_library_host_code_under_sanitizers():
    runtime = sanitized_build.clang_asan_runtime()
    if not runtime or not os.path.exists(sanitized_build.HIPCC):
        pytest.skip("no hipcc or clang ASan runtime")
    lib = sanitized_build.build_library()
    out = _run_child(["tests/test_abi_host.py", "tests/test_group_plan_host.py"],
                     {"LD_PRELOAD": runtime, "SPCONV_LIB_PATH": lib})
    assert " passed" in out
