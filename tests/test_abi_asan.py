"""The C-ABI tests (tests/test_abi.py) again, against the host-side
AddressSanitizer build of the library (libgdn_asan.so: every host function
instrumented, built by gated_deltanet_state_amd.build with asan=True), in a
child process with the sanitizer runtime preloaded.  Any out-of-bounds
access, use after free or bad free in the argument checks, workspace sizing,
error reporting or the launch plumbing up to the first HIP call aborts the
child and fails this test.  CPU only: the calls here never reach a kernel."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_address_sanitizer():
    from gated_deltanet_state_amd import build
    if not os.path.exists(build.LIB_ASAN):
        pytest.skip("libgdn_asan.so is not built (python -m gated_deltanet_state_amd.build --asan)")
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["GDN_TEST_LIB"] = build.LIB_ASAN
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, "ABI tests failed under AddressSanitizer"
    assert "ERROR: AddressSanitizer" not in r.stderr
