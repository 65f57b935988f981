"""The C ABI's host code under AddressSanitizer and UBSan: the CPU ABI and
binding tests rerun, in a child process, against a host-only sanitized build
of the library (tests/host_asan.py), with the sanitizer runtime preloaded.
Any heap overflow, use after free or undefined behaviour (signed overflow,
misaligned access, out-of-range shift) in argument validation, layout or
split planning aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

import host_asan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_bindings_under_asan_ubsan():
    if host_asan.hipcc() is None:
        pytest.skip("hipcc not available")
    rt = host_asan.asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    lib = host_asan.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "library is not instrumented"
    env = dict(os.environ)
    env.update(KVQ_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
