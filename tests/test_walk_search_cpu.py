"""Host check of the gather kernels' request search (interpolation guess,
galloping, bisection) against a linear scan, on random workspace_starts with
empty, one-row and long requests (tests/pins/walk_search.cpp)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def test_find_request_matches_linear_scan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "walk_search")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-o", exe,
                    os.path.join(ROOT, "tests", "pins", "walk_search.cpp")], check=True,
                   capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
