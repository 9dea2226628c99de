"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: api.hip (every
entry point's argument validation, workspace sizing and launch set-up) rebuilt with both
sanitizers (`python -m kv_cache_compressed_amd.build --host-sanitize`), loaded with the ASan
runtime preloaded, and the whole C-ABI test file run against it in a child process. Any heap or
stack overflow, use after free or undefined behaviour (signed overflow, bad shift, misaligned
access, ...) on those paths aborts the child. Needs no GPU: none of these calls reaches a launch."""
import os
import subprocess
import sys

import pytest

from kv_cache_compressed_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = build.build_host_sanitized(verbose=False)
    env = dict(os.environ, LD_PRELOAD=rt, VC_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
