"""The ABI layer's host code (argument validation, workspace sizing, status
messages) under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU ABI
tests run again, in a child process with the sanitizer runtime preloaded,
against a build of libsparda whose api.cpp carries host-only instrumentation
(kv_block_selection_amd.build.build_host_sanitized)."""

import os
import subprocess
import sys

import pytest

from kv_block_selection_amd import build as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_clean_under_host_sanitizers():
    try:
        lib = kb.build_host_sanitized()
        runtime = kb.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=runtime, SPARDA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the instrumented library, with the sanitizer runtime live
    probe = ("import ctypes, kv_block_selection_amd as k; k.load(); "
             f"assert k.LIB_PATH == {lib!r}; ctypes.CDLL(None).__asan_init; print('instrumented')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "instrumented" in r.stdout, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"], env=env,
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
