"""The row clamp of the direct global->LDS tile copies, checked on the CPU.

The copy kernels read row min(row0 + r, N - 1) for every tile row r; a
block-sparse tile can start past N - 1.  tests/tile_copy_check.cpp includes
the device header and exercises the helper on the host over every tile
start, row and matrix height up to 400.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_copy_row_clamp(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "tile_copy_check"
    src = os.path.join(ROOT, "tests", "tile_copy_check.cpp")
    inc = os.path.join(ROOT, "io_aware_tiled_05_amd", "csrc")
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", inc, src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
