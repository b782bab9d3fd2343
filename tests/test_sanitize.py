"""The host code of the C ABI (argument validation, size helpers, status strings) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every rejection path by
tests/sanitize/abi_driver.cpp.  CPU only: no call in the driver reaches a kernel launch."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SCRIPT = os.path.join(HERE, "sanitize", "build_and_run.sh")


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not available")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    r = subprocess.run(["bash", SCRIPT, str(tmp_path / "asan")], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi driver ok" in r.stdout
