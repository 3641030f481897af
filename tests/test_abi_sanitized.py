"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The library is rebuilt with the host-side sanitizers (``build(sanitize=True)``; device
code as usual) into a temporary directory, and ``tests/test_abi.py`` -- every entry point
fed valid, invalid, misaligned and out-of-range arguments, all rejected before any
launch -- runs against it in a child process with the clang ASan runtime preloaded. Any
sanitizer report aborts the child.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    from exact_io_aware_flash_amd import build as B

    try:
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build(sanitize=True, out=str(tmp_path / "libfa_san.so"))
    env = dict(os.environ, LD_PRELOAD=runtime, FA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
