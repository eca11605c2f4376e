"""The host side of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

build.build_sanitized() compiles runtime.cpp (handle tables, argument and
config validation, weight and workspace planning, the graph cache, the
ternary pack/unpack helpers, the fault injector) with both sanitizers; the
host ABI tests then run in a child process that loads that build with the
sanitizer runtime preloaded.  Any invalid access or undefined behaviour aborts
the child, so the test fails.  (The paper, §III-C: a request returns the chunk
"or an error" -- every failure has to come back as a status, never a crash.)
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from prefix_cache_flow_amd import build
    try:
        lib = build.build_sanitized(verbose=False)
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.fail(f"sanitized build failed: {e}")
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host runtime is not instrumented"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "VLA_LIBRARY": lib,
        # Python itself is not instrumented and keeps memory until exit: no leak report
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "HIP_VISIBLE_DEVICES": "",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_host.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized run failed (exit {r.returncode}):\n{tail}"
    assert "passed" in r.stdout
