"""The C ABI's host-side validation, workspace planning and error strings built with
AddressSanitizer and UndefinedBehaviorSanitizer (host pass only) and exercised by a small
driver that makes no GPU call (CPU only)."""
import shutil
import subprocess

import pytest


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_validation_under_asan_and_ubsan():
    from long_context_sparse_stage0_amd import sanitize_build
    exe = sanitize_build.build_sanitized()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env={"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
                            "PATH": "/usr/bin:/bin"})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ok: 0 failure(s)" in out
    assert "AddressSanitizer" not in out and "runtime error" not in out
