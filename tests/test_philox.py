"""The kernels' Philox4x32-10, checked on the CPU.

tests/philox_check.cpp includes the device header and compares the
generator used by the dropout kernels with the published known-answer
vectors (the oracle's independent implementation is checked against the
same vectors in test_oracle_dropout.py).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_device_philox_known_answers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "philox_check"
    src = os.path.join(ROOT, "tests", "philox_check.cpp")
    inc = os.path.join(ROOT, "io_aware_tiled_05_amd", "csrc")
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", inc, src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
