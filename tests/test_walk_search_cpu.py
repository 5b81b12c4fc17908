"""Host check of the gather kernels' request searches (interpolation guess,
galloping, bisection; the six-step bisection used for batches up to 64)
against a linear scan, on random workspace_starts with empty, one-row and
long requests; termination inside [0, batch) on invalid workspace_starts; and
the row-address bounds that turn a bad walk into a zero row
(tests/pins/walk_search.cpp)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def test_request_search_and_row_bounds(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "walk_search")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-o", exe,
                    os.path.join(ROOT, "tests", "pins", "walk_search.cpp")], check=True,
                   capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
