"""The swizzled LDS tile layout of the 16-bit kernels, checked on the CPU.

tests/lds_swizzle_check.cpp includes the device header and checks, for
d = 32, 64, 96 and 128, that the copy map and the read offsets are inverse
bijections and that the two read patterns of a tile (16 rows of one chunk
column; 4 rows x 4 chunks for the transpose reads) each touch all 16 bank
groups once.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lds_tile_layout_is_a_conflict_free_bijection(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "lds_swizzle_check"
    src = os.path.join(ROOT, "tests", "lds_swizzle_check.cpp")
    inc = os.path.join(ROOT, "io_aware_tiled_05_amd", "csrc")
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", inc, src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
