"""CPU bounds check of the forward kernel's global-memory index arithmetic.

tests/geometry_check.hip includes the kernel's own geometry helpers
(bit_quantized_exact_amd/csrc/fwd_geometry.h) and enumerates every global
address the kernel forms, for tail shapes and large shapes, on the host.
No GPU is used."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_forward_kernel_addresses_stay_in_bounds(tmp_path):
    exe = tmp_path / "geometry_check"
    subprocess.check_call([
        HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950",
        "-I", os.path.join(ROOT, "bit_quantized_exact_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
        os.path.join(ROOT, "tests", "geometry_check.hip"), "-o", str(exe)],
        stderr=subprocess.DEVNULL)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "0 errors" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_decode_kernel_addresses_stay_in_bounds(tmp_path):
    exe = tmp_path / "decode_geometry_check"
    subprocess.check_call([
        HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950",
        "-I", os.path.join(ROOT, "bit_quantized_exact_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
        os.path.join(ROOT, "tests", "decode_geometry_check.hip"), "-o", str(exe)],
        stderr=subprocess.DEVNULL)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "0 errors" in r.stdout
