"""The host logic of libcalibatt.so under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the host-sanitized variant of the library (the device code is the
ordinary gfx950 code; only the host compilation is instrumented), then runs
the C-ABI tests (argument checks, list-view validation) against it in a child
process with the ASan runtime preloaded. Any sanitizer report ends the child
with a non-zero status.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_calibatt_build", os.path.join(ROOT, "calibrated_block_sparse_skiplist_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_under_address_and_ub_sanitizers():
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    lib = b.build_sanitized()
    env = dict(os.environ)
    env["LD_PRELOAD"] = b.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["CALIBATT_LIB"] = lib
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                          "-p", "no:cacheprovider", "-m", "not gpu"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
