"""Build the GPU converter sweep used by tests/test_gpu_converters.py:

    tests/pins/libconverter_sweep.so   hipcc, gfx950, the library's own flags
                                       (the kernels run gcache_device.h's
                                       conversion helpers)
    tests/pins/libconverter_check.so   gcc, the oracle's flags, linked to
                                       oracle/libgcache_oracle.so

    python tests/pins/build.py [-v]

Test infrastructure only; __graft_entry__.build() runs it so that the GPU
tests find both libraries built beforehand.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SWEEP_SRC = os.path.join(HERE, "converter_sweep.hip")
CHECK_SRC = os.path.join(HERE, "converter_check.c")
SWEEP_LIB = os.path.join(HERE, "libconverter_sweep.so")
CHECK_LIB = os.path.join(HERE, "libconverter_check.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
C_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-Wall", "-Wextra", "-Werror", "-pthread"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")


def build(verbose: bool = False):
    tmp = SWEEP_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-o", tmp, SWEEP_SRC], verbose)
    os.replace(tmp, SWEEP_LIB)
    tmp = CHECK_LIB + ".tmp"
    _run([os.environ.get("CC", shutil.which("gcc") or "cc"), *C_FLAGS, "-o", tmp, CHECK_SRC,
          "-L", os.path.join(ROOT, "oracle"), "-lgcache_oracle", "-lm",
          "-Wl,-rpath,$ORIGIN/../../oracle"], verbose)
    os.replace(tmp, CHECK_LIB)
    return SWEEP_LIB, CHECK_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
