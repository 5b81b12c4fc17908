"""Compile the CPU oracle (plain C, gcc) into oracle/libgcache_oracle.so.

Test infrastructure only.  Flags keep every binary32 operation a single IEEE
rounding: no fused multiply-add contraction, no fast-math, no x87 excess
precision (SSE2 arithmetic on x86-64).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gcache_oracle.c")
LIB = os.path.join(HERE, "libgcache_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    """Compile the oracle library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only if the library is missing or older than its sources."""
    srcs = [SRC, os.path.join(HERE, "gcache_oracle.h")]
    if not os.path.exists(LIB) or any(os.path.getmtime(s) > os.path.getmtime(LIB) for s in srcs):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
