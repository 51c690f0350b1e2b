"""The workgroup -> (tile, head) map of the kernels, checked on the CPU.

tests/workgroup_map_check.cpp includes the device header and checks that
the snake-ordered map is a permutation of the grid for ragged grids (a
partial last dispatch round included), keeps a head's tiles on one XCD, and
balances causal work over compute units.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_workgroup_map_is_a_balanced_permutation(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "workgroup_map_check"
    src = os.path.join(ROOT, "tests", "workgroup_map_check.cpp")
    inc = os.path.join(ROOT, "io_aware_tiled_05_amd", "csrc")
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", inc, src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
