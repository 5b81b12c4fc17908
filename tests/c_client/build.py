"""Build tests/c_client/gcache_client, a plain C99 program that links
libgcache.so and the HIP runtime and calls the library only through
include/gcache.h (gcc, no hipcc: nothing in it runs on the GPU itself).

    python tests/c_client/build.py
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "gather_concat_cache_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "gcache_client")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC", shutil.which("gcc") or "cc")
    tmp = EXE + ".tmp"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
           os.path.join(HERE, "gcache_client.c"), "-o", tmp,
           "-L", PKG, "-lgcache", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gather_concat_cache_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
