"""The host-side validation of the C ABI (argument checks, workspace sizing, the overlap
sweep) under AddressSanitizer and UndefinedBehaviorSanitizer: tests/test_abi.py run in a
child process against the host-only sanitized build of the library, with the sanitizer
runtime preloaded.  Any out-of-bounds access, use after free or undefined behaviour in
that code aborts the child.  CPU only."""
import os
import subprocess
import sys

import pytest

from attention_guided_eviction_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_asan_and_ubsan():
    try:
        runtime = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(BKV_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
