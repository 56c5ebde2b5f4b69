"""The C ABI's host layer (argument checks, workspace layout, the fixed
scratch lookup) under AddressSanitizer and UndefinedBehaviorSanitizer: the
ABI tests (no GPU) run in a subprocess against a build of the library whose
host code is instrumented; any sanitizer report fails them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_address_and_ub_sanitizers():
    sys.path.insert(0, os.path.join(ROOT, "block_diffusion_drafter_rmsnorm_amd"))
    import importlib
    b = importlib.import_module("build")
    try:
        lib = b.build_sanitized(verbose=False)
        rt = b.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(f"no sanitizer build here: {e}")
    env = dict(os.environ)
    env.update(DFLASH_LIBRARY=lib, LD_PRELOAD=rt, LD_LIBRARY_PATH=os.path.dirname(rt),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
