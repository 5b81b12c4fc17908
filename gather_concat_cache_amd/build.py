"""Build libgcache.so (HIP, gfx950 only) in-tree with hipcc.

    python gather_concat_cache_amd/build.py [-v]

Flags:
  --offload-arch=gfx950            the only target
  -ffp-contract=off                every binary32 multiply / divide rounds once,
                                   exactly as the reference rules are written
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                   no packed-FP32 VALU instructions
  (no fast-math: IEEE division and denormals are part of the bit-exact contract)
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgcache.so")
SOURCES = ["ds_mla_kernels.hip", "nvfp4_kv_kernels.hip", "sparse_index.hip", "gcache_abi.hip"]
# measurement helper beside the library (include/gcache_bench.h), loaded by bench.py only
BENCH_LIB = os.path.join(PKG, "libgcache_bench.so")
BENCH_SOURCES = ["bench_ceiling.hip"]
HEADERS = ["gcache_device.h", "gcache_internal.h"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unknown-warning-option", "-I", os.path.join(ROOT, "include")]


def _compile(src, obj, verbose):
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected and dropped, anything else is shown.
    noise = ("packed-fp32-ops", "unknown target feature", "warning generated")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def _link(lib, objs, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libgcache.so (and the
    measurement helper libgcache_bench.so)."""
    objdir = os.path.join(ROOT, "_build", "gcache")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        list(ex.map(lambda so: _compile(*so, verbose), zip(srcs, objs)))
    _link(LIB, objs[:len(SOURCES)], verbose)
    _link(BENCH_LIB, objs[len(SOURCES):], verbose)
    return LIB


def source_digest() -> str:
    """sha256 of every source and header the library is built from (the
    kernels, their headers and the C ABI header)."""
    import hashlib
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "gcache.h")]:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stale() -> bool:
    """True when the library is missing or older than any source."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "gcache.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
