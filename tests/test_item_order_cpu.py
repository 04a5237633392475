"""The grouped GEMMs' work-item order (blocked_tile, device_common.h) is a bijection onto an
expert's M x N tiles for every shape and block height: compiled for the host and run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_routed_topk_amd", "csrc")


def test_blocked_tile_is_a_bijection(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "blocked_tile_check"
    src = os.path.join(ROOT, "tests", "cpp", "blocked_tile_check.cpp")
    r = subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--cuda-host-only", "-I", CSRC, src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
