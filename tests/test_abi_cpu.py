"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/gcache.h declares, its host-only helpers return the format
constants, and invalid arguments are rejected on the host before any HIP
call (no kernel is ever launched here)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "gcache.h")


@pytest.fixture(scope="module")
def lib():
    from gather_concat_cache_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import gather_concat_cache_amd as g
    return g.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gcache_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == sorted([
        "gcache_entry_bytes", "gcache_nvfp4_full_dim", "gcache_status_string",
        "gcache_cache_write_nvfp4_ds_mla", "gcache_cache_write_fp8_ds_mla",
        "gcache_cache_gather_upconvert_nvfp4_ds_mla", "gcache_cache_gather_upconvert_fp8_ds_mla",
        "gcache_cache_gather_bf16", "gcache_context_chunk_plan", "gcache_context_chunk",
        "gcache_convert_req_index_to_global_index",
        "gcache_nvfp4_kv_split_layout", "gcache_nvfp4_kv_split_layout_hnd", "gcache_reshape_and_cache_nvfp4",
        "gcache_gather_upconvert_nvfp4_kv", "gcache_time_next_launch"]), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by libgcache.so"


def test_timing_hook_is_host_only(lib):
    """Arming and disarming the kernel timing hook touches no device."""
    assert lib.gcache_time_next_launch(None, None) == 0


def test_host_helpers(lib):
    g = load_golden("formats.json")
    assert lib.gcache_entry_bytes(0) == g["nvfp4_ds_mla_entry_bytes"]
    assert lib.gcache_entry_bytes(1) == g["fp8_ds_mla_entry_bytes"]
    assert lib.gcache_entry_bytes(7) == -1
    for hs, fd in g["full_dim"].items():
        assert lib.gcache_nvfp4_full_dim(int(hs)) == fd
    assert lib.gcache_nvfp4_full_dim(24) == -1 and lib.gcache_nvfp4_full_dim(0) == -1
    assert lib.gcache_status_string(0) == b"ok"
    assert b"gfx950" in lib.gcache_status_string(-4)


def test_split_layout_matches_the_oracle_layout(lib, orc):
    import gather_concat_cache_amd as g
    for bs, H, hs in ((16, 8, 128), (1, 1, 16), (64, 3, 80)):
        mine = g.nvfp4_kv_split_layout(bs, H, hs)
        ref = orc.kv_layout_split(bs, H, hs)
        assert {n: getattr(mine, n) for n, _ in mine._fields_} == ref.as_dict()
    with pytest.raises(g.GcacheError) as e:
        g.nvfp4_kv_split_layout(16, 8, 100)
    assert e.value.status == -2


# Fake device addresses: never dereferenced, because every call below fails
# validation before the library touches the device.
A16 = 0x10000


def _write(lib, fn, **kw):
    a = dict(kv_c=A16, k_pe=A16, cache=A16, slots=A16, T=4, kvs=512, kps=64, nb=2, bs=64,
             bstr=64 * 352, estr=352, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["kv_c"], a["k_pe"], a["cache"], a["slots"], a["T"], a["kvs"], a["kps"],
                            a["nb"], a["bs"], a["bstr"], a["estr"], a["stream"])


@pytest.mark.parametrize("fn,eb", [("gcache_cache_write_nvfp4_ds_mla", 352),
                                   ("gcache_cache_write_fp8_ds_mla", 656)])
def test_write_argument_validation(lib, fn, eb):
    kw = dict(bstr=64 * eb, estr=eb)
    assert _write(lib, fn, T=0, kv_c=None, **kw) == 0                 # empty: no-op
    assert _write(lib, fn, T=-1, **kw) == -2
    assert _write(lib, fn, kv_c=None, **kw) == -1
    assert _write(lib, fn, slots=None, **kw) == -1
    assert _write(lib, fn, kvs=500, **kw) == -2
    assert _write(lib, fn, kps=32, **kw) == -2
    assert _write(lib, fn, bs=0, **kw) == -2
    assert _write(lib, fn, bstr=64 * eb, estr=eb - 16) == -2
    assert _write(lib, fn, bstr=63 * eb, estr=eb) == -2               # entries of a block overlap
    assert _write(lib, fn, nb=-1, **kw) == -2
    assert _write(lib, fn, kv_c=A16 + 8, **kw) == -3
    assert _write(lib, fn, kvs=516, **kw) == -3
    assert _write(lib, fn, cache=A16 + 4, **kw) == -3
    assert _write(lib, fn, bstr=64 * eb + 8, estr=eb) == -3


def _gather(lib, fn, **kw):
    a = dict(src=A16, dst=A16, total=10, ds=576, bt=A16, bts=8, ws=A16, ss=A16, B=2, nb=4, bs=64,
             bstr=64 * 352, estr=352, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["src"], a["dst"], a["total"], a["ds"], a["bt"], a["bts"], a["ws"], a["ss"],
                            a["B"], a["nb"], a["bs"], a["bstr"], a["estr"], a["stream"])


@pytest.mark.parametrize("fn,eb", [("gcache_cache_gather_upconvert_nvfp4_ds_mla", 352),
                                   ("gcache_cache_gather_upconvert_fp8_ds_mla", 656)])
def test_gather_argument_validation(lib, fn, eb):
    kw = dict(bstr=64 * eb, estr=eb)
    assert _gather(lib, fn, total=0, src=None, **kw) == 0
    assert _gather(lib, fn, total=-3, **kw) == -2
    assert _gather(lib, fn, dst=None, **kw) == -1
    assert _gather(lib, fn, bt=None, **kw) == -1
    assert _gather(lib, fn, ws=None, **kw) == -1
    assert _gather(lib, fn, B=0, **kw) == -2
    assert _gather(lib, fn, ds=512, **kw) == -2
    assert _gather(lib, fn, bts=0, **kw) == -2
    assert _gather(lib, fn, total=1 << 31, **kw) == -2
    assert _gather(lib, fn, dst=A16 + 2, **kw) == -3
    assert _gather(lib, fn, ds=580, **kw) == -3
    assert _gather(lib, fn, src=A16 + 8, **kw) == -3


def test_perhead_argument_validation(lib):
    import gather_concat_cache_amd as g
    L = g.nvfp4_kv_split_layout(16, 8, 128)
    f = lib.gcache_reshape_and_cache_nvfp4

    def call(**kw):
        a = dict(key=A16, value=A16, kts=1024, khs=128, vts=1024, vhs=128, cache=A16, slots=A16, T=4, H=8,
                 hs=128, nb=4, bs=16, L=C.byref(L), ks=A16, vs=A16, stream=None)
        a.update(kw)
        return f(a["key"], a["value"], a["kts"], a["khs"], a["vts"], a["vhs"], a["cache"], a["slots"], a["T"],
                 a["H"], a["hs"], a["nb"], a["bs"], a["L"], a["ks"], a["vs"], a["stream"])
    assert call(T=0, key=None) == 0
    assert call(key=None) == -1
    assert call(L=None) == -1
    assert call(ks=None) == -1
    assert call(hs=120) == -2
    assert call(hs=2048) == -2
    assert call(H=0) == -2
    assert call(kts=1020) == -3
    assert call(key=A16 + 2) == -3
    bad = g.NvFp4KvLayout(**{n: getattr(L, n) for n, _ in L._fields_})
    bad.data_head_stride = 60
    assert call(L=C.byref(bad)) == -3
    bad.data_head_stride = -64
    assert call(L=C.byref(bad)) == -2


def test_binding_exposes_the_c_names(lib):
    """Every device entry point (and the layout/size helpers) is reachable
    from Python under its C name; the host-only chunk planner and the HND
    layout are reached through context_chunks and
    nvfp4_kv_split_layout(hnd=True), gcache_status_string through the
    exception text."""
    import gather_concat_cache_amd as g
    wrapped_elsewhere = {"gcache_status_string", "gcache_context_chunk_plan", "gcache_context_chunk",
                         "gcache_nvfp4_kv_split_layout_hnd"}
    for n in declared_functions():
        if n not in wrapped_elsewhere:
            assert callable(getattr(g, n, None)), f"{n} has no Python counterpart"


def test_bench_helper_library():
    """libgcache_bench.so (the same-mix copy bench.py measures as a ceiling)
    loads, exports what include/gcache_bench.h declares, and rejects bad
    arguments before touching the device."""
    from gather_concat_cache_amd import build
    if not os.path.exists(build.BENCH_LIB):
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gcache_bench.h")).read(), flags=re.S)
    assert sorted(set(re.findall(r"\b(gcache_[a-z0-9_]+)\s*\(", text))) == ["gcache_bench_copy_mix",
                                                                           "gcache_bench_empty_grid"]
    blib = C.CDLL(build.BENCH_LIB)
    f = blib.gcache_bench_copy_mix
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
    f.restype = C.c_int
    assert f(None, None, 0, 352, 1152, 16, 256, None) == 0           # empty: no-op
    assert f(None, A16, 10, 352, 1152, 16, 256, None) == -1
    assert f(A16, A16, 10, 350, 1152, 16, 256, None) == -2
    assert f(A16, A16, 10, 352, 1168, 16, 256, None) == -2
    assert f(A16, A16, -1, 352, 1152, 16, 256, None) == -2
    assert f(A16, A16, 10, 352, 1152, 0, 256, None) == -2            # no rows per group
    assert f(A16, A16, 10, 352, 1152, 16, 96, None) == -2            # not a whole number of waves
    assert f(A16, A16, 10, 1152, 352, 17, 1024, None) == -2          # more than 18 KiB staged
    assert f(A16 + 8, A16, 10, 352, 1152, 16, 256, None) == -3
    e = blib.gcache_bench_empty_grid
    e.argtypes = [C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    e.restype = C.c_int
    for groups, threads in ((0, 256), (1 << 31, 256), (1, 0), (1, 96), (1, 1088)):
        assert e(groups, threads, None, None, None) == -2
