"""The C ABI checks under AddressSanitizer (host code only, no GPU): tests/run_abi_asan.py
builds the host-instrumented library and runs tests/test_abi.py on it; a sanitizer report
aborts that run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_clean_under_address_sanitizer():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "run_abi_asan.py")],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
