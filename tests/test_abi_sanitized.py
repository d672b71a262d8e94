"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the ABI host sources are built with g++ and sanitizers into a
host-check library whose kernel launchers are stubs, and the CPU ABI tests run
against it in a child process with the ASan runtime preloaded.  Any sanitizer
report fails the child."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "host_abi"))


def _runtime(name):
    if shutil.which("g++") is None:
        return None
    p = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_host_code_is_sanitizer_clean(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    import build_hostcheck

    lib = build_hostcheck.build(str(tmp_path / "libwq_hostcheck.so"))
    env = dict(os.environ)
    env.update({
        "WQ_LIB": lib,
        "LD_PRELOAD": asan,
        # the interpreter itself is not instrumented: leak checking would
        # report its own allocations
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out
