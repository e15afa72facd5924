"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: libhr_asan.so (host pass built with both sanitizers, GPU code as
usual) runs every validation test of tests/test_abi.py in a child process with
the ASan runtime preloaded; any sanitizer report fails."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_validation_under_asan_and_ubsan():
    from codebook_decode_amd import build as b
    lib = b.build(verbose=False, asan=True)
    try:
        env = dict(os.environ, HR_LIB=lib, LD_PRELOAD=b.asan_runtime(),
                   ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=540)
        out = r.stdout + r.stderr
        assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
        assert r.returncode == 0, out[-4000:]
    finally:
        if os.path.exists(lib):
            os.remove(lib)
