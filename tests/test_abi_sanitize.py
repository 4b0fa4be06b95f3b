"""The library's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/sanitize/build_and_run.sh builds the host code with both sanitizers (device code
as usual, never launched) into a driver that calls every entry point with rejected or empty-work
arguments, sizes up to the int64 extremes included. A sanitizer report or an unexpected status
fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("g++") is None,
                    reason="needs hipcc and g++")
def test_abi_checks_under_asan_ubsan():
    out = os.path.join(ROOT, "_build", "sanitize")
    r = subprocess.run(["bash", os.path.join(ROOT, "tests", "sanitize", "build_and_run.sh"), out],
                       capture_output=True, text=True, timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "all calls rejected or empty as expected" in r.stdout, report
