"""The oracle's pin suites again, against a build of the oracle's C source
with AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc), in a
child process: an out-of-bounds access or an undefined operation inside the
oracle would otherwise only show as a wrong expected value."""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

PIN_SUITES = ["tests/test_oracle_ops.py", "tests/test_context_chunks_cpu.py", "tests/test_sparse_index_cpu.py",
              "tests/test_kv_views_cpu.py"]


def test_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    so = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-fexcess-precision=standard", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"), "-o", so,
                    os.path.join(ROOT, "oracle", "gcache_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, GCACHE_ORACLE_LIB=so, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: the child's pytest must not capture stderr, where the reports go
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PIN_SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    lines = out.splitlines()
    first = next((i for i, l in enumerate(lines) if "runtime error" in l or "AddressSanitizer" in l), None)
    tail = "\n".join(lines[first:first + 30] if first is not None else lines[-40:])
    assert r.returncode == 0, tail
    assert "runtime error" not in out and "AddressSanitizer" not in out, tail
    assert "passed" in r.stdout, tail
