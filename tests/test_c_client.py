"""libgcache.so driven from a plain C99 program (tests/c_client/gcache_client.c)
through include/gcache.h alone: hipMalloc'd buffers, a stream of its own,
status codes.  The CPU test runs its host-only calls and rejected calls and
checks them against the golden format constants and the oracle's own layout
and chunk planner; the GPU test has it write and gather seeded caches, and
compares every cache byte and output bit with the oracle."""
import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import ROOT, load_golden

HERE = os.path.join(ROOT, "tests", "c_client")
EXE = os.path.join(HERE, "gcache_client")


def _load_build():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_gcache_c_client_build", os.path.join(HERE, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def client_cpu():
    """On the CPU the client is (re)built here when missing or older than its
    source or the library it links."""
    from gather_concat_cache_amd import build
    if build.stale():
        build.build()
    deps = [os.path.join(HERE, "gcache_client.c"), build.LIB, os.path.join(ROOT, "include", "gcache.h")]
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(d) for d in deps):
        _load_build().build()
    return EXE


def _host_lines(exe):
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    return dict(line.split("=", 1) for line in r.stdout.splitlines())


def test_host_entry_points_from_c(client_cpu, orc):
    out = _host_lines(client_cpu)
    g = load_golden("formats.json")
    assert int(out["entry_bytes_nvfp4"]) == g["nvfp4_ds_mla_entry_bytes"]
    assert int(out["entry_bytes_fp8"]) == g["fp8_ds_mla_entry_bytes"]
    assert int(out["full_dim_128"]) == g["full_dim"]["128"]
    assert int(out["full_dim_24"]) == -1
    names = ["data_offset", "data_token_stride", "data_head_stride", "scale_offset", "scale_token_stride",
             "scale_head_stride", "side_stride", "block_stride"]
    for key, hnd in (("split_nhd_16_8_128", False), ("split_hnd_16_8_128", True)):
        want = orc.kv_layout_split(16, 8, 128, hnd=hnd).as_dict()
        assert [int(v) for v in out[key].split(",")] == [want[n] for n in names], key
    assert int(out["split_bad_head"]) == -2

    chunk_rows, chunks = orc.context_chunks([700, 0, 1500], 1000, 64)
    assert out["chunk_plan"] == f"{chunk_rows},{len(chunks)}"
    for i, (ss, ws, total) in enumerate(chunks):
        assert out[f"chunk_{i}"] == ",".join(map(str, ss)) + "|" + ",".join(map(str, ws)) + f"|{total}"
    assert int(out["chunk_out_of_range"]) == -2 and int(out["chunk_null_output"]) == -1
    assert int(out["write_null_input"]) == -1
    assert int(out["write_short_entry"]) == -2
    assert int(out["write_misaligned"]) == -3
    assert int(out["gather_no_requests"]) == -2
    assert int(out["gather_empty"]) == 0
    assert "gfx950" in out["status_unsupported"]


def _cases():
    import synth
    w1, _, g_all = synth.tiny_round_trip()
    yield "tiny_round_trip-all-blocks", w1, g_all
    rng = np.random.default_rng(61)
    nb, bs = 40, 64
    w = synth.random_write(62, 1500, nb, bs, 30)
    g = synth.prefill_gather(rng, "c-client-prefill", 5, 100, 450, nb, bs, 8)
    yield "random-write-5-requests", w, g


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_roundtrip_from_c(orc, tmp_path, fmt):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build() (or tests/c_client/build.py) first")
    eb = 352 if fmt == "nvfp4" else 656
    owrite = orc.write_nvfp4_ds_mla if fmt == "nvfp4" else orc.write_fp8_ds_mla
    ogather = orc.gather_nvfp4_ds_mla if fmt == "nvfp4" else orc.gather_fp8_ds_mla
    for name, w, g in _cases():
        print(f"C client round trip: {fmt} {name}", flush=True)
        d = tmp_path / f"{fmt}-{name}"
        d.mkdir()
        T = w.slot_mapping.shape[0]
        np.ascontiguousarray(w.kv_c, np.uint16).tofile(d / "kv_c.bin")
        np.ascontiguousarray(w.k_pe, np.uint16).tofile(d / "k_pe.bin")
        np.ascontiguousarray(w.slot_mapping, np.int64).tofile(d / "slots.bin")
        np.ascontiguousarray(g.block_table, np.int32).tofile(d / "block_table.bin")
        np.ascontiguousarray(g.workspace_starts, np.int32).tofile(d / "ws.bin")
        np.ascontiguousarray(g.seq_starts, np.int32).tofile(d / "ss.bin")
        B, maxb = g.block_table.shape
        r = subprocess.run([EXE, "roundtrip", fmt, str(d), str(T), str(w.num_blocks), str(w.block_size), str(B),
                            str(maxb), str(g.total_tokens)], capture_output=True, text=True, timeout=120)
        sys.stdout.write(r.stdout)
        assert r.returncode == 0, r.stderr
        want = np.full(w.num_blocks * w.block_size * eb, 0xA5, np.uint8)
        owrite(w.kv_c, w.k_pe, want, w.slot_mapping, w.num_blocks, w.block_size)
        got = np.fromfile(d / "cache.bin", np.uint8)
        assert np.array_equal(got, want), f"{fmt} {name}: cache bytes differ from the oracle"
        ref = ogather(want, g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, w.num_blocks,
                      w.block_size)
        out = np.fromfile(d / "out.bin", np.uint16).reshape(g.total_tokens, 576)
        assert np.array_equal(out, ref), f"{fmt} {name}: gathered rows differ from the oracle"
        # the gather's kernel-bound events (gcache_time_next_launch) recorded a duration
        ms = [float(l.split("=", 1)[1]) for l in r.stdout.splitlines() if l.startswith("gather_kernel_ms=")]
        assert len(ms) == (1 if g.total_tokens > 0 else 0) and all(0.0 < m < 1000.0 for m in ms), r.stdout
