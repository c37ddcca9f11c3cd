"""The workgroup -> work-item maps of the HIP kernels (host-side build of sla_tiles.hpp)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_xcd_maps_are_balanced_bijections(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    exe = tmp_path / "remap_check"
    src = os.path.join(ROOT, "tests", "remap_check.cpp")
    inc = os.path.join(ROOT, "block_sparse_linear_02_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{inc}", src,
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
