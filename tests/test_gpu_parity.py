"""GPU parity: every HIP entry point, called through the C ABI (Python
binding), against the CPU oracle on the same seeded inputs -- bit-exact on
every cache byte (sentinel-filled, so untouched bytes are checked too) and
every bf16 output bit.  Sizes span several workgroups and ragged tails; the
full-size workloads run in the launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_same, dev, filled_cache, host

pytestmark = pytest.mark.gpu

NV, F8 = 352, 656


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gather_concat_cache_amd as gc
    return gc


def _ds_pair(fmt):
    import gather_concat_cache_amd as gc
    if fmt == "nvfp4":
        return NV, gc.cache_write_nvfp4_ds_mla, gc.cache_gather_upconvert_nvfp4_ds_mla
    return F8, gc.cache_write_fp8_ds_mla, gc.cache_gather_upconvert_fp8_ds_mla


def _orc_ds(orc, fmt):
    if fmt == "nvfp4":
        return orc.write_nvfp4_ds_mla, orc.gather_nvfp4_ds_mla
    return orc.write_fp8_ds_mla, orc.gather_fp8_ds_mla


def _cache_view(flat, nb, bs, bstr, estr):
    return torch.as_strided(flat, (nb, bs, estr), (bstr, estr, 1))


def run_ds_write(orc, fmt, kv_c, k_pe, slots, nb, bs, bstr=None, estr=None, fill=0xA5,
                 kv_dev=None, pe_dev=None):
    """GPU write vs oracle write into identically pre-filled flat caches.
    Returns the oracle's cache (the expected bytes)."""
    eb, gwrite, _ = _ds_pair(fmt)
    owrite, _ = _orc_ds(orc, fmt)
    estr = estr or eb
    bstr = bstr or bs * estr
    want = np.full(nb * bstr, fill, np.uint8)
    owrite(kv_c, k_pe, want, slots, nb, bs, bstr, estr)
    flat = filled_cache((nb * bstr,), fill)
    gwrite(kv_dev if kv_dev is not None else dev(kv_c), pe_dev if pe_dev is not None else dev(k_pe),
           _cache_view(flat, nb, bs, bstr, estr), dev(slots))
    torch.cuda.synchronize()
    assert_same(host(flat), want, f"{fmt} write cache bytes")
    return want, flat


def run_ds_gather(orc, fmt, cache_np, cache_dev, gcase, nb, bs, bstr=None, estr=None, dst_stride=576,
                  seq_starts=True):
    eb, _, ggather = _ds_pair(fmt)
    _, ogather = _orc_ds(orc, fmt)
    estr = estr or eb
    bstr = bstr or bs * estr
    ss = gcase.seq_starts if seq_starts else None
    want = np.full((gcase.total_tokens, dst_stride), 0x7FC1, np.uint16)
    ogather(cache_np, gcase.total_tokens, gcase.block_table, gcase.workspace_starts, ss, nb, bs, bstr,
            estr, dst=want)
    dst = dev(np.full((gcase.total_tokens, dst_stride), 0x7FC1, np.uint16))
    ggather(_cache_view(cache_dev, nb, bs, bstr, estr), dst, dev(gcase.block_table),
            dev(gcase.workspace_starts), None if ss is None else dev(ss))
    torch.cuda.synchronize()
    assert_same(host(dst), want, f"{fmt} gather ({gcase.name})")


# ---------------------------------------------------------------------------
# nvfp4_ds_mla and fp8_ds_mla
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_tiny_round_trip(g, orc, fmt):
    w, g_tok, g_all = synth.tiny_round_trip()
    want, flat = run_ds_write(orc, fmt, w.kv_c, w.k_pe, w.slot_mapping, 8, 64)
    for gc_ in (g_tok, g_all):
        run_ds_gather(orc, fmt, want, flat, gc_, 8, 64)


def test_rounding_order_hand_vectors(g, orc):
    """The hand-derived rounding-order cases through the kernels: the fp8
    write multiplies by the reciprocal scale, the fp8 gather rounds the
    binary32 product to bf16, the per-head scale is (amax / 6) / gs and the
    per-head dequant rounds twice.  Each result is compared with the
    fixture's value and with the oracle."""
    from conftest import load_golden
    from test_oracle_ops import fp8_gather_rounding_entry, golden_gs
    f8 = load_golden("fp8_ds_mla_vectors.json")
    w = f8["write_rounding"]
    row = np.zeros((1, 512), np.float32)
    row[0, :len(w["values_head"])] = w["values_head"]
    kv_c = synth.bf16_bits(row)
    k_pe = np.zeros((1, 64), np.uint16)
    want, flat = run_ds_write(orc, "fp8", kv_c, k_pe, np.zeros(1, np.int64), 1, 1, fill=0)
    e = host(flat)
    assert [f"{c:#04x}" for c in e[:len(w["codes_head"])]] == w["codes_head"]
    assert e[512:516].tobytes().hex() == w["scale_le"]
    one = synth.GatherCase("one row", np.zeros((1, 1), np.int32), np.zeros(1, np.int32),
                           np.zeros(1, np.int32), 1, 1, 1, np.ones(1, np.int64))
    run_ds_gather(orc, "fp8", want, flat, one, 1, 1)
    r = f8["gather_rounding"]
    entry = fp8_gather_rounding_entry(r)
    flat = dev(entry)
    run_ds_gather(orc, "fp8", entry, flat, one, 1, 1)
    _, _, ggather = _ds_pair("fp8")
    dst = dev(np.zeros((1, 576), np.uint16))
    ggather(_cache_view(flat, 1, 1, F8, F8), dst, dev(one.block_table), dev(one.workspace_starts), None)
    torch.cuda.synchronize()
    assert [f"{b:#06x}" for b in host(dst)[0, :len(r["codes"])]] == r["dequant_bf16"]

    # per-head: one token, one head of 16 values; data at 0, scale byte at 8
    kw = dict(data_offset=0, data_token_stride=8, data_head_stride=8, scale_offset=8, scale_token_stride=1,
              scale_head_stride=1, side_stride=16, block_stride=32)
    L_orc, L_gpu = orc.KvLayout(**kw), g.NvFp4KvLayout(**kw)
    for h in load_golden("perhead_vectors.json")["heads"]:
        gs = golden_gs(h)
        key = synth.bf16_bits(np.array(h["values"], np.float32).reshape(1, 1, 16))
        run_kv(orc, g, key, key, np.zeros(1, np.int64), 1, 1, L_orc, L_gpu, gs, gs)
        flat = filled_cache((32,), 0xA5)
        cache5 = torch.as_strided(flat, (1, 2, 1, 1, 9), (32, 16, 9, 9, 1))
        gs_d = torch.tensor([gs], dtype=torch.float32, device="cuda")
        g.reshape_and_cache_nvfp4(dev(key), dev(key), cache5, dev(np.zeros(1, np.int64)), gs_d, gs_d,
                                  layout=L_gpu)
        ko = torch.zeros((1, 1, 16), dtype=torch.bfloat16, device="cuda")
        vo = torch.zeros_like(ko)
        g.gather_upconvert_nvfp4_kv(cache5, ko, vo, dev(np.zeros((1, 1), np.int32)), dev(np.zeros(1, np.int32)),
                                    gs_d, gs_d, layout=L_gpu)
        torch.cuda.synchronize()
        c = host(flat)
        for side in (0, 1):
            assert c[16 * side:16 * side + 8].tobytes().hex() == h["data"], h["name"]
            assert c[16 * side + 8] == int(h["scale_byte"], 16), h["name"]
        k = host(ko)[0, 0]
        assert np.array_equal(host(vo)[0, 0], k), h["name"]
        if "dequant_bits" in h:
            assert [f"{b:#06x}" for b in k] == h["dequant_bits"], h["name"]


def test_kernel_timing_hook(g, orc):
    """gcache_time_next_launch binds the next launch's own begin and end to
    two events: the kernel still computes the same bytes, the elapsed time is
    positive and no longer than events recorded around the call, a rejected
    call leaves the hook armed, and the launch after the timed one is plain."""
    import ctypes
    import os
    hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_NOW)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    ev = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e.value)
    w = synth.decode_batch_write()
    eb, gwrite, _ = _ds_pair("nvfp4")
    want = np.full(w.num_blocks * w.block_size * eb, 0xA5, np.uint8)
    orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, want, w.slot_mapping, w.num_blocks, w.block_size)
    kv, pe, sl = dev(w.kv_c), dev(w.k_pe), dev(w.slot_mapping)
    flat = filled_cache((w.num_blocks * w.block_size * eb,), 0xA5)
    cache = flat.view(w.num_blocks, w.block_size, eb)
    g.time_next_launch(ev[0], ev[1])
    odd_stride = torch.zeros((w.kv_c.shape[0], 513), dtype=torch.bfloat16, device="cuda")[:, :512]
    with pytest.raises(g.GcacheError):                       # rejected (row stride 513): hook kept
        gwrite(odd_stride, pe, cache, sl)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    gwrite(kv, pe, cache, sl)                                # the timed launch
    b.record()
    gwrite(kv, pe, cache, sl)                                # plain launch: the events keep the first
    torch.cuda.synchronize()
    assert_same(host(flat), want, "write under the timing hook")
    t = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1])) == 0
    assert 0.0 < t.value <= a.elapsed_time(b), (t.value, a.elapsed_time(b))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_decode_batch_write(g, orc, fmt):
    w = synth.decode_batch_write()
    run_ds_write(orc, fmt, w.kv_c, w.k_pe, w.slot_mapping, w.num_blocks, w.block_size)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_ragged_strided_non_pow2_block(g, orc, fmt):
    """Odd token count, kv_c / k_pe as slices of one [T, 584] buffer, block
    size 48 (the generic division path), padded entries (entry_stride >
    entry) and gaps between blocks; gathers with empty requests, a wider dst
    row stride, with and without seq_starts."""
    rng = np.random.default_rng(77)
    eb = NV if fmt == "nvfp4" else F8
    T, nb, bs = 1001, 30, 48
    estr = eb + 32
    bstr = bs * estr + 256
    buf = synth.bf16_bits(rng.standard_normal((T, 584), dtype=np.float32)
                          * np.exp(rng.standard_normal((T, 1), dtype=np.float32)))
    kv_c, k_pe = buf[:, :512], buf[:, 520:584]
    slots = synth.padded_slots(rng, nb * bs, T, 37)
    bdev = dev(buf)
    want, flat = run_ds_write(orc, fmt, kv_c, k_pe, slots, nb, bs, bstr, estr,
                              kv_dev=bdev[:, :512], pe_dev=bdev[:, 520:584])
    # requests: lengths with empty requests in between, arbitrary seq_starts
    L = np.array([100, 0, 333, 1, 0, 200, 47, 480, 0], np.int64)
    s = np.array([5, 0, 100, 0, 0, 199, 0, 3, 0], np.int64)
    rows = np.where(L > 0, L - s, 0)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((9, 12), -1, np.int32)
    pos = 0
    for b in range(9):
        n = -(-int(L[b]) // bs)
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    assert pos <= nb
    ws = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int32)
    gcase = synth.GatherCase("ragged", bt, ws, s.astype(np.int32), int(rows.sum()), nb, bs, L)
    assert gcase.total_tokens % 16 != 0
    run_ds_gather(orc, fmt, want, flat, gcase, nb, bs, bstr, estr, dst_stride=600)
    g0 = synth.GatherCase("ragged-no-starts", bt, ws, np.zeros(9, np.int32), int(rows.sum()), nb, bs, L)
    run_ds_gather(orc, fmt, want, flat, g0, nb, bs, bstr, estr, seq_starts=False)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_edge_cases(g, orc, fmt):
    eb, gwrite, ggather = _ds_pair(fmt)
    rng = np.random.default_rng(3)
    kv_c = synth.bf16_bits(rng.standard_normal((5, 512), dtype=np.float32))
    k_pe = synth.bf16_bits(rng.standard_normal((5, 64), dtype=np.float32))
    # all padding: nothing is written
    run_ds_write(orc, fmt, kv_c, k_pe, np.full(5, -1, np.int64), 2, 16)
    # one token, into the very last slot
    run_ds_write(orc, fmt, kv_c[:1], k_pe[:1], np.array([31], np.int64), 2, 16)
    # zero tokens / zero rows: no-ops that touch nothing
    flat = filled_cache((2 * 16 * eb,), 0x33)
    gwrite(dev(kv_c[:0]), dev(k_pe[:0]), _cache_view(flat, 2, 16, 16 * eb, eb), dev(np.zeros(0, np.int64)))
    ggather(_cache_view(flat, 2, 16, 16 * eb, eb), dev(np.zeros((0, 576), np.uint16)),
            dev(np.zeros((1, 2), np.int32)), dev(np.zeros(1, np.int32)))
    torch.cuda.synchronize()
    assert np.all(host(flat) == 0x33)
    # zero and negative-zero blocks, saturating magnitudes, subnormal scales
    x = np.zeros((4, 512), np.float32)
    x[1, :16] = -0.0
    x[2] = rng.standard_normal(512).astype(np.float32) * np.float32(3e4)
    x[3] = rng.standard_normal(512).astype(np.float32) * np.float32(1e-4)
    run_ds_write(orc, fmt, synth.bf16_bits(x), k_pe[:4], np.arange(4, dtype=np.int64), 1, 4)
    with pytest.raises(g.GcacheError):                       # misaligned row stride
        gwrite(dev(np.zeros((2, 516), np.uint16))[:, :512], dev(k_pe[:2]),
               _cache_view(flat, 2, 16, 16 * eb, eb), dev(np.zeros(2, np.int64)))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_full_size_prefill_write_and_gather(g, orc, fmt):
    """The benchmark's workloads: the 524288-token (nvfp4) / 1048576-token
    (fp8) pre-fill writes and the 16- / 32-request prefill gathers, whole
    cache and whole workspace compared."""
    w = synth.nvfp4_prefill_write() if fmt == "nvfp4" else synth.fp8_prefill_write()
    gcase = synth.nvfp4_prefill_gather() if fmt == "nvfp4" else synth.fp8_prefill_gather()
    want, flat = run_ds_write(orc, fmt, w.kv_c, w.k_pe, w.slot_mapping, w.num_blocks, w.block_size)
    del w
    run_ds_gather(orc, fmt, want, flat, gcase, gcase.num_blocks, gcase.block_size)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_request_counts_around_one_wave(g, orc, fmt):
    """Batches of 1, 63, 64 and 65 requests (the gather resolves requests
    with cross-lane reads up to 64 and searches memory beyond) and one
    single-row request per token of the decode batch (4014 requests)."""
    w = synth.decode_batch_write()
    want, flat = run_ds_write(orc, fmt, w.kv_c, w.k_pe, w.slot_mapping, w.num_blocks, w.block_size)
    run_ds_gather(orc, fmt, want, flat, synth.per_token_gather("per-token", w.slot_mapping, w.num_blocks,
                                                               w.block_size), w.num_blocks, w.block_size)
    rng = np.random.default_rng(64)
    for B in (1, 63, 64, 65):
        gc_ = synth.prefill_gather(rng, f"B{B}", B, 1, 700, w.num_blocks, w.block_size, 12)
        run_ds_gather(orc, fmt, want, flat, gc_, w.num_blocks, w.block_size)


def _walk_slots(total, bt, ws, ss, bs, nb):
    """Slot read by each workspace row (linear scan over the requests), -1
    where the position leaves the block-table row or names a block outside
    [0, nb)."""
    out = np.full(total, -1, np.int64)
    for r in range(total):
        b = max(i for i in range(len(ws)) if ws[i] <= r)
        pos = int(ss[b]) + r - int(ws[b])
        if pos < 0 or pos // bs >= bt.shape[1]:
            continue
        blk = int(bt[b, pos // bs])
        if 0 <= blk < nb:
            out[r] = blk * bs + pos % bs
    return out


def _bad_metadata(nb, bs):
    """Three requests over a 4-column block table: a block id past the cache,
    a negative block id, and a request whose positions run past the row."""
    bt = np.array([[0, 1, nb, 2], [3, -5, 4, 5], [5, 4, 3, 2]], np.int32)
    ws = np.array([0, 57, 121], np.int32)
    ss = np.array([3, 0, 50], np.int32)
    return bt, ws, ss, 151


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_out_of_range_metadata(g, orc, fmt):
    """Slot ids outside [0, num_blocks * block_size) are skipped like padding;
    gather rows whose walk leaves the block-table row or the cache come back
    as zeros and every other row is exact."""
    eb, gwrite, ggather = _ds_pair(fmt)
    _, ogather = _orc_ds(orc, fmt)
    rng = np.random.default_rng(91)
    nb, bs, T = 6, 16, 80
    kv_c = synth.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    k_pe = synth.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    raw = slots.copy()
    raw[[3, 10, 40, 77]] = [nb * bs, -7, 1 << 40, nb * bs + 5]
    clean = raw.copy()
    clean[[3, 10, 40, 77]] = -1
    want = np.full(nb * bs * eb, 0xA5, np.uint8)
    _orc_ds(orc, fmt)[0](kv_c, k_pe, want, clean, nb, bs, bs * eb, eb)
    flat = filled_cache((nb * bs * eb,), 0xA5)
    gwrite(dev(kv_c), dev(k_pe), _cache_view(flat, nb, bs, bs * eb, eb), dev(raw))
    torch.cuda.synchronize()
    assert_same(host(flat), want, f"{fmt} write with out-of-range slots")

    bt, ws, ss, total = _bad_metadata(nb, bs)
    rs = _walk_slots(total, bt, ws, ss, bs, nb)
    assert 0 < int((rs < 0).sum()) < total
    exp = np.zeros((total, 576), np.uint16)
    ok = rs >= 0
    pt = synth.per_token_gather("valid rows", rs[ok], nb, bs)
    exp[ok] = ogather(want, pt.total_tokens, pt.block_table, pt.workspace_starts, pt.seq_starts, nb, bs)
    dst = dev(np.full((total, 576), 0x7FC1, np.uint16))
    ggather(_cache_view(flat, nb, bs, bs * eb, eb), dst, dev(bt), dev(ws), dev(ss))
    torch.cuda.synchronize()
    assert_same(host(dst), exp, f"{fmt} gather with out-of-range metadata")


def _bf16_gather_case(orc, g, cache_bits, gcase, nb, bs, estr_el, bt=None, zero_rows=None):
    """GPU BF16 comparator gather vs the oracle on bf16 cache bits
    [nb, bs, estr_el] (rows with an invalid walk expected as zeros)."""
    bt = gcase.block_table if bt is None else bt
    flat = cache_bits.reshape(-1).view(np.uint8)
    if zero_rows is None:
        want = orc.gather_bf16(flat, gcase.total_tokens, bt, gcase.workspace_starts, gcase.seq_starts, nb,
                               bs, bs * estr_el * 2, estr_el * 2)
    else:
        want = zero_rows
    cache_dev = dev(cache_bits)[:, :, :576] if estr_el > 576 else dev(cache_bits)
    dst = dev(np.full((gcase.total_tokens, 576), 0x7FC1, np.uint16))
    g.cache_gather_bf16(cache_dev, dst, dev(bt), dev(gcase.workspace_starts), dev(gcase.seq_starts))
    torch.cuda.synchronize()
    assert_same(host(dst), want, f"bf16 gather ({gcase.name})")


def test_bf16_comparator_gather(g, orc):
    """The BF16 comparator copies the walked rows bit for bit (random bits,
    NaN patterns included): prefill-like requests, 65 requests (memory
    search), padded entries, and zero rows for an invalid walk."""
    rng = np.random.default_rng(55)
    nb, bs = 80, 16
    for estr_el in (576, 600):
        cache = rng.integers(0, 1 << 16, size=(nb, bs, estr_el), dtype=np.uint16)
        for B in (3, 65):
            gc_ = synth.prefill_gather(rng, f"bf16-B{B}", B, 0, 9, nb, bs, 1)
            _bf16_gather_case(orc, g, cache, gc_, nb, bs, estr_el)
        gc_ = synth.prefill_gather(rng, "bf16-long", 4, 20, 150, nb, bs, 10)
        _bf16_gather_case(orc, g, cache, gc_, nb, bs, estr_el)
    # invalid walk: expected rows from a per-row oracle gather, zeros elsewhere
    cache = rng.integers(0, 1 << 16, size=(6, 16, 576), dtype=np.uint16)
    bt, ws, ss, total = _bad_metadata(6, 16)
    rs = _walk_slots(total, bt, ws, ss, 16, 6)
    ok = rs >= 0
    pt = synth.per_token_gather("valid rows", rs[ok], 6, 16)
    exp = np.zeros((total, 576), np.uint16)
    exp[ok] = orc.gather_bf16(cache.reshape(-1).view(np.uint8), pt.total_tokens, pt.block_table,
                              pt.workspace_starts, pt.seq_starts, 6, 16)
    gc_ = synth.GatherCase("bf16-bad-metadata", bt, ws, ss, total, 6, 16, None)
    _bf16_gather_case(orc, g, cache, gc_, 6, 16, 576, zero_rows=exp)


def test_bf16_comparator_gather_full_size(g, orc):
    """The nvfp4 prefill gather's requests over a bf16 cache of the same
    geometry (8192 blocks x 64 x 1152 B): every row compared."""
    gcase = synth.nvfp4_prefill_gather()
    cache = synth.normal_bf16_rows(1013, 0, gcase.num_blocks * gcase.block_size, 576)
    _bf16_gather_case(orc, g, cache.reshape(gcase.num_blocks, gcase.block_size, 576), gcase,
                      gcase.num_blocks, gcase.block_size, 576)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8", "bf16"])
def test_chunked_context_gather(g, orc, fmt):
    """Whole contexts gathered through a small workspace chunk by chunk equal
    the oracle's one-shot gather of the same contexts, row for row
    (contexts of 0, 1, one block, many blocks plus a tail; 9 chunks)."""
    rng = np.random.default_rng(123)
    nb, bs = 128, 16
    lens = np.array([0, 1, 16, 700, 130, 1000, 64], np.int32)
    B = lens.shape[0]
    nblk = -(-lens // bs)
    assert int(nblk.sum()) <= nb
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, int(nblk.max())), -1, np.int32)
    pos = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += int(nblk[b])
    full = synth.GatherCase("full", bt, np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32),
                            np.zeros(B, np.int32), int(lens.sum()), nb, bs, lens)
    if fmt == "bf16":
        cache_bits = rng.integers(0, 1 << 16, size=(nb, bs, 576), dtype=np.uint16)
        cache_np = cache_bits.reshape(-1).view(np.uint8)
        cache_dev = dev(cache_bits)
        want = orc.gather_bf16(cache_np, full.total_tokens, bt, full.workspace_starts, full.seq_starts, nb, bs)
        gather = g.cache_gather_bf16
    else:
        eb, _, gather = _ds_pair(fmt)
        T = nb * bs
        kv_c = synth.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
        k_pe = synth.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
        cache_np = np.zeros(T * eb, np.uint8)
        owrite, ogather = _orc_ds(orc, fmt)
        owrite(kv_c, k_pe, cache_np, np.arange(T, dtype=np.int64), nb, bs)
        cache_dev = dev(cache_np).view(nb, bs, eb)
        want = ogather(cache_np, full.total_tokens, bt, full.workspace_starts, full.seq_starts, nb, bs)
    workspace = torch.zeros((7 * 48 + 5, 576), dtype=torch.bfloat16, device="cuda")
    c, plan = g.context_chunks(lens, workspace.shape[0], bs)
    assert c == 48 and len(plan) == 21
    got = [[] for _ in range(B)]
    for i, rows in g.gather_context_chunked(gather, cache_dev, workspace, dev(bt), lens):
        h = host(rows)
        ss, ws, tot = plan[i]
        ends = np.concatenate([ws[1:], [tot]])
        for b in range(B):
            got[b].append(h[ws[b]:ends[b]])
    got = np.concatenate([np.concatenate(x) if x else np.zeros((0, 576), np.uint16) for x in got])
    assert_same(got, want, f"chunked {fmt} gather")


def test_sparse_index_conversion(g, orc):
    """Hand vectors, random rows on the element path (topk % 4 != 0,
    strided input and output) and the vector path, invalid entries, the
    length check, and the full decode-batch shape (4096 x 2048)."""
    from conftest import load_golden
    gv = load_golden("sparse_index_vectors.json")
    for case in gv["cases"]:
        out = g.convert_req_index_to_global_index(dev(np.array(gv["req_id"], np.int32)),
                                                  dev(np.array(gv["token_indices"], np.int32)),
                                                  dev(np.array(gv["block_table"], np.int32)),
                                                  gv["block_size"], case["num_blocks"])
        assert host(out).tolist() == case["out"]
    rng = np.random.default_rng(71)
    # (topk, 16-byte path, extra out columns): partial and several waves per row on
    # both paths, and a strided but aligned output on the 16-byte path
    for K, vec, extra in ((37, False, 3), (256, True, 0), (300, False, 3), (1024, True, 0), (1500, True, 4),
                          (4, True, 4), (2052, True, 0)):
        B, mb, bs, nb, T = 5, 9, 16, 60, 50
        bt = rng.integers(-2, nb + 3, size=(B, mb)).astype(np.int32)
        req = rng.integers(-1, B + 2, size=T).astype(np.int32)
        ti = rng.integers(-3, mb * bs + 5, size=(T, K)).astype(np.int32)
        want = orc.convert_req_index(req, ti, bt, bs, nb)
        wide = np.zeros((T, K + 5), np.int32)
        wide[:, :K] = ti
        ti_dev = dev(ti) if vec else dev(wide)[:, :K]
        out = torch.full((T, K + extra), 7, dtype=torch.int32, device="cuda")
        got = g.convert_req_index_to_global_index(dev(req), ti_dev, dev(bt), bs, nb,
                                                  out=out if extra else None)
        torch.cuda.synchronize()
        assert_same(host(got)[:, :K], want, f"sparse index K={K}")
        if extra:
            assert np.all(host(out)[:, K:] == 7)          # bytes past topk untouched
    with pytest.raises(g.GcacheError):                    # req_id one longer than the rows
        g.convert_req_index_to_global_index(dev(np.zeros(6, np.int32)), dev(np.zeros((5, 8), np.int32)),
                                            dev(np.zeros((1, 1), np.int32)), 16, 1)
    req, idx, bt, bs, nb = synth.sparse_index_case()
    got = g.convert_req_index_to_global_index(dev(req), dev(idx), dev(bt), bs, nb)
    assert_same(host(got), orc.convert_req_index(req, idx, bt, bs, nb), "sparse index 4096 x 2048")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("bs", [1, 3, 512])
def test_extreme_block_sizes(g, orc, fmt, bs):
    """Block sizes 1 (every token its own block), 3 (odd, division path) and
    512 (more rows per block than a gather tile): write and gather."""
    rng = np.random.default_rng(500 + bs)
    nb = max(4, 600 // bs)
    T = min(nb * bs, 333)
    kv_c = synth.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    k_pe = synth.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    slots = synth.padded_slots(rng, nb * bs, T, 7)
    want, flat = run_ds_write(orc, fmt, kv_c, k_pe, slots, nb, bs)
    run_ds_gather(orc, fmt, want, flat, synth.per_token_gather("per-token", slots, nb, bs), nb, bs)
    hi = bs * (nb // 3)                    # three requests always fit the cache
    gc_ = synth.prefill_gather(rng, "prefill", 3, 1, hi, nb, bs, nb // 3)
    run_ds_gather(orc, fmt, want, flat, gc_, nb, bs)


@pytest.mark.parametrize("H,hs", [(1, 1024), (32, 16), (2, 48)])
def test_perhead_extreme_heads(g, orc, H, hs):
    """Largest head (1024 values), smallest head (16), one head, many heads,
    and a head size that is not a power of two."""
    rng = np.random.default_rng(H * 1000 + hs)
    nb, bs, T = 12, 16, 150
    key, value, slots = _kv_case(rng, T, H, hs, nb, bs, 4)
    L = orc.kv_layout_split(bs, H, hs)
    run_kv(orc, g, key, value, slots, nb, bs, L, None, synth.global_scale(key), synth.global_scale(value))


# ---------------------------------------------------------------------------
# per-head NVFP4 K/V
# ---------------------------------------------------------------------------
def _kv_case(rng, T, H, hs, nb, bs, pad):
    mag_k = rng.uniform(0.1, 10, (1, H, 1)).astype(np.float32)
    key = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * mag_k)
    value = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * np.float32(0.05))
    slots = synth.padded_slots(rng, nb * bs, T, pad)
    return key, value, slots


def run_kv(orc, g, key, value, slots, nb, bs, L_orc, L_gpu, ks, vs, key_dev=None, value_dev=None,
           out_hnd=False):
    T, H, hs = key.shape
    side = max(L_orc.side_stride, 1)
    size = nb * L_orc.block_stride
    want = np.full(size, 0xA5, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, want, slots, nb, bs, L_orc, ks, vs)
    flat = filled_cache((size,), 0xA5)
    fd = hs // 2 + hs // 16
    cache5 = torch.as_strided(flat, (nb, 2, bs, H, fd), (L_orc.block_stride, side, H * fd, fd, 1))
    ks_d = torch.tensor([ks], dtype=torch.float32, device="cuda")
    vs_d = torch.tensor([vs], dtype=torch.float32, device="cuda")
    g.reshape_and_cache_nvfp4(key_dev if key_dev is not None else dev(key),
                              value_dev if value_dev is not None else dev(value),
                              cache5, dev(slots), ks_d, vs_d, layout=L_gpu)
    torch.cuda.synchronize()
    assert_same(host(flat), want, "per-head write cache bytes")
    gcase = synth.per_token_gather("kv", slots, nb, bs)
    ok, ov = orc.gather_upconvert_nvfp4_kv(want, gcase.total_tokens, gcase.block_table,
                                           gcase.workspace_starts, gcase.seq_starts, H, hs, nb, bs,
                                           L_orc, ks, vs)
    n = gcase.total_tokens
    if out_hnd:   # outputs as [H, n, hs] memory viewed as [n, H, hs]
        kb = torch.zeros((H, n, hs), dtype=torch.bfloat16, device="cuda")
        vb = torch.zeros((H, n, hs), dtype=torch.bfloat16, device="cuda")
        ko, vo = kb.permute(1, 0, 2), vb.permute(1, 0, 2)
    else:
        ko = torch.zeros((n, H, hs), dtype=torch.bfloat16, device="cuda")
        vo = torch.zeros((n, H, hs), dtype=torch.bfloat16, device="cuda")
    g.gather_upconvert_nvfp4_kv(cache5, ko, vo, dev(gcase.block_table), dev(gcase.workspace_starts),
                                ks_d, vs_d, seq_starts=dev(gcase.seq_starts), layout=L_gpu)
    torch.cuda.synchronize()
    assert_same(host(ko.contiguous()), ok, "per-head gather K")
    assert_same(host(vo.contiguous()), ov, "per-head gather V")


@pytest.mark.parametrize("layout", ["split", "interleaved-rows"])
def test_perhead_full_workload(g, orc, layout):
    """The per-head workload at full size (8192 tokens, 8 heads of 128,
    4096 blocks of 16), every byte and output bit: the default split layout
    (direct kernels) and [data | scale] rows per (token, head) (576-byte
    runs per token and side, the staged kernels), as the bench times them."""
    w, _ = synth.perhead_write_gather()
    H, hs, bs = 8, 128, w.block_size
    if layout == "split":
        L_orc, L_gpu = orc.kv_layout_split(bs, H, hs), None
    else:
        fd = hs // 2 + hs // 16
        kw = dict(data_offset=0, data_token_stride=H * fd, data_head_stride=fd, scale_offset=hs // 2,
                  scale_token_stride=H * fd, scale_head_stride=fd, side_stride=bs * H * fd,
                  block_stride=2 * bs * H * fd)
        L_orc, L_gpu = orc.KvLayout(**kw), g.NvFp4KvLayout(**kw)
    run_kv(orc, g, w.key, w.value, w.slot_mapping, w.num_blocks, bs, L_orc, L_gpu, w.k_scale, w.v_scale)


@pytest.mark.parametrize("variant", ["interleaved", "interleaved-3heads", "hnd", "hnd-split", "odd-head-size",
                                     "strided-input"])
def test_perhead_layouts(g, orc, variant):
    """Layouts: interleaved [data | scales] rows (4 heads: 16-byte aligned
    token runs, the staged kernels; 3 heads: 216-byte runs, the direct
    kernels), HND orders, a head size of 80, strided inputs."""
    seed = {"interleaved": 41, "interleaved-3heads": 47, "hnd": 42, "hnd-split": 45, "odd-head-size": 43,
            "strided-input": 44}[variant]
    rng = np.random.default_rng(seed)
    # head size 80: 5 scale blocks and 10 chunks per head (the non-power-of-two paths)
    # interleaved [data | scales] rows keep 8-byte data alignment at head size 128 (72-byte rows)
    H, hs, nb, bs = {"odd-head-size": (3, 80, 20, 16), "interleaved": (4, 128, 16, 16),
                     "interleaved-3heads": (3, 128, 16, 16)}.get(variant, (4, 64, 16, 16))
    T = 157
    key, value, slots = _kv_case(rng, T, H, hs, nb, bs, 9)
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    fd = hs // 2 + hs // 16
    if variant.startswith("interleaved"):   # each (token, head) row is [data | scales]
        kw = dict(data_offset=0, data_token_stride=H * fd, data_head_stride=fd, scale_offset=hs // 2,
                  scale_token_stride=H * fd, scale_head_stride=fd, side_stride=bs * H * fd,
                  block_stride=2 * bs * H * fd)
    elif variant == "hnd":              # split layout with heads outermost inside a side
        kw = dict(data_offset=0, data_token_stride=hs // 2, data_head_stride=bs * hs // 2,
                  scale_offset=bs * H * hs // 2, scale_token_stride=hs // 16,
                  scale_head_stride=bs * hs // 16, side_stride=bs * H * fd, block_stride=2 * bs * H * fd)
    elif variant == "hnd-split":        # each side's layout from the library's and the oracle's HND helpers
        kw = orc.kv_layout_split(bs, H, hs, hnd=True).as_dict()
    else:
        kw = orc.kv_layout_split(bs, H, hs).as_dict()
    L_orc, L_gpu = orc.KvLayout(**kw), g.NvFp4KvLayout(**kw)
    if variant == "hnd-split":
        L_gpu = g.nvfp4_kv_split_layout(bs, H, hs, hnd=True)
    kd = vd = None
    if variant == "strided-input":      # key / value as slices of a wider [T, H, hs + 16] buffer
        big = np.zeros((T, H, hs + 16), np.uint16)
        big[:, :, :hs] = key
        kd = dev(big)[:, :, :hs]
        big2 = np.zeros((T, H, hs + 16), np.uint16)
        big2[:, :, :hs] = value
        vd = dev(big2)[:, :, :hs]
    run_kv(orc, g, key, value, slots, nb, bs, L_orc, L_gpu, ks, vs, kd, vd, out_hnd=(variant == "hnd"))


def _prefill_requests(rng, B, nb, bs, long_len, empties):
    """B requests over a shuffle of the nb blocks: lengths U[1, 520] plus one
    request of long_len positions, gather starts U[0, L] (a start at L makes
    the request empty) with the requests in `empties` forced empty and a few
    starts inside the first block; workspace_starts = exclusive cumsum."""
    L = rng.integers(1, 521, size=B).astype(np.int64)
    L[B // 2] = long_len
    s = rng.integers(0, L + 1).astype(np.int64)
    s[empties] = L[empties]
    s[1], s[2] = 0, min(5, int(L[2]))
    nblk = -(-L // bs)
    assert nblk.sum() <= nb
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((B, int(nblk.max()) + 2), -1, np.int32)
    pos = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    rows = L - s
    ws = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int32)
    return synth.GatherCase("prefill walk", bt, ws, s.astype(np.int32), int(rows.sum()), nb, bs, L)


@pytest.mark.parametrize("layout", ["nhd-split", "hnd-split", "rows"])
def test_perhead_prefill_walks(g, orc, layout):
    """The per-head gather on prefill-shaped walks (multi-row requests read
    from seq_starts, empty requests, one long request spanning many blocks):
    48 requests, about 8k rows, 8 heads of 128, over a cache whose every slot
    was written by the per-head write; NHD and HND split layouts and
    [data | scale] rows (the staged kernels).  Every byte and output bit
    against the oracle, with and without seq_starts."""
    rng = np.random.default_rng({"nhd-split": 61, "hnd-split": 62, "rows": 63}[layout])
    H, hs, bs, nb, B = 8, 128, 16, 1280, 48
    fd = hs // 2 + hs // 16
    T = nb * bs
    key, value, _ = _kv_case(rng, T, H, hs, nb, bs, 0)
    slots = rng.permutation(T).astype(np.int64)
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    if layout == "rows":
        kw = dict(data_offset=0, data_token_stride=H * fd, data_head_stride=fd, scale_offset=hs // 2,
                  scale_token_stride=H * fd, scale_head_stride=fd, side_stride=bs * H * fd,
                  block_stride=2 * bs * H * fd)
        L_orc, L_gpu = orc.KvLayout(**kw), g.NvFp4KvLayout(**kw)
    else:
        L_orc = orc.kv_layout_split(bs, H, hs, hnd=layout == "hnd-split")
        L_gpu = g.nvfp4_kv_split_layout(bs, H, hs, hnd=layout == "hnd-split")
    size = nb * L_orc.block_stride
    want = np.full(size, 0xA5, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, want, slots, nb, bs, L_orc, ks, vs)
    flat = filled_cache((size,), 0xA5)
    cache5 = torch.as_strided(flat, (nb, 2, bs, H, fd), (L_orc.block_stride, L_orc.side_stride, H * fd, fd, 1))
    ks_d = torch.tensor([ks], dtype=torch.float32, device="cuda")
    vs_d = torch.tensor([vs], dtype=torch.float32, device="cuda")
    g.reshape_and_cache_nvfp4(dev(key), dev(value), cache5, dev(slots), ks_d, vs_d, layout=L_gpu)
    torch.cuda.synchronize()
    assert_same(host(flat), want, f"per-head write ({layout})")
    gc_ = _prefill_requests(rng, B, nb, bs, 3000, [3, 17, 40])
    assert 5000 < gc_.total_tokens < 12000
    for ss in (gc_.seq_starts, None):
        ok, ov = orc.gather_upconvert_nvfp4_kv(want, gc_.total_tokens, gc_.block_table, gc_.workspace_starts,
                                               ss, H, hs, nb, bs, L_orc, ks, vs)
        ko = torch.full((gc_.total_tokens, H, hs), 7.0, dtype=torch.bfloat16, device="cuda")
        vo = torch.full((gc_.total_tokens, H, hs), 7.0, dtype=torch.bfloat16, device="cuda")
        g.gather_upconvert_nvfp4_kv(cache5, ko, vo, dev(gc_.block_table), dev(gc_.workspace_starts), ks_d, vs_d,
                                    seq_starts=None if ss is None else dev(ss), layout=L_gpu)
        torch.cuda.synchronize()
        what = f"per-head prefill gather ({layout}, {'with' if ss is not None else 'without'} seq_starts)"
        assert_same(host(ko), ok, what + " K")
        assert_same(host(vo), ov, what + " V")


def test_perhead_out_of_range_metadata(g, orc):
    """Per-head write skips out-of-range slot ids; the per-head gather writes
    zero K and V rows where the walk leaves the block table or the cache."""
    rng = np.random.default_rng(92)
    H, hs, nb, bs, T = 2, 64, 6, 16, 80
    key, value, _ = _kv_case(rng, T, H, hs, nb, bs, 0)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    raw = slots.copy()
    raw[[0, 33, 79]] = [nb * bs, -9, 1 << 41]
    clean = raw.copy()
    clean[[0, 33, 79]] = -1
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    L = orc.kv_layout_split(bs, H, hs)
    size = nb * L.block_stride
    want = np.full(size, 0xA5, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, want, clean, nb, bs, L, ks, vs)
    flat = filled_cache((size,), 0xA5)
    fd = hs // 2 + hs // 16
    cache5 = torch.as_strided(flat, (nb, 2, bs, H, fd), (L.block_stride, L.side_stride, H * fd, fd, 1))
    ks_d = torch.tensor([ks], dtype=torch.float32, device="cuda")
    vs_d = torch.tensor([vs], dtype=torch.float32, device="cuda")
    g.reshape_and_cache_nvfp4(dev(key), dev(value), cache5, dev(raw), ks_d, vs_d)
    torch.cuda.synchronize()
    assert_same(host(flat), want, "per-head write with out-of-range slots")

    bt, ws, ss, total = _bad_metadata(nb, bs)
    rs = _walk_slots(total, bt, ws, ss, bs, nb)
    ok = rs >= 0
    pt = synth.per_token_gather("valid rows", rs[ok], nb, bs)
    vk, vv = orc.gather_upconvert_nvfp4_kv(want, pt.total_tokens, pt.block_table, pt.workspace_starts,
                                           pt.seq_starts, H, hs, nb, bs, L, ks, vs)
    ek = np.zeros((total, H, hs), np.uint16)
    ev = np.zeros((total, H, hs), np.uint16)
    ek[ok], ev[ok] = vk, vv
    ko = dev(np.full((total, H, hs), 0x7FC1, np.uint16))
    vo = dev(np.full((total, H, hs), 0x7FC1, np.uint16))
    g.gather_upconvert_nvfp4_kv(cache5, ko, vo, dev(bt), dev(ws), ks_d, vs_d, seq_starts=dev(ss))
    torch.cuda.synchronize()
    assert_same(host(ko), ek, "per-head gather K with out-of-range metadata")
    assert_same(host(vo), ev, "per-head gather V with out-of-range metadata")


def test_perhead_split_views_on_device(g, orc):
    """The split views of a device cache written through the HND layout hold
    the bytes the oracle writes (data as uint8, scales as float8_e4m3fn)."""
    rng = np.random.default_rng(46)
    H, hs, nb, bs, T = 4, 64, 10, 16, 100
    key, value, slots = _kv_case(rng, T, H, hs, nb, bs, 5)
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    L = orc.kv_layout_split(bs, H, hs, hnd=True)
    fd = hs // 2 + hs // 16
    want = np.zeros(nb * 2 * bs * H * fd, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, want, slots, nb, bs, L, ks, vs)
    cache5 = torch.zeros((nb, 2, bs, H, fd), dtype=torch.uint8, device="cuda")
    Lg = g.nvfp4_kv_split_layout(bs, H, hs, hnd=True)
    g.reshape_and_cache_nvfp4(dev(key), dev(value), cache5, dev(slots),
                              torch.tensor([ks], dtype=torch.float32, device="cuda"),
                              torch.tensor([vs], dtype=torch.float32, device="cuda"), layout=Lg)
    torch.cuda.synchronize()
    dv, sv = g.nvfp4_kv_split_views(cache5, H, hs, Lg)
    dh, sh = g.nvfp4_kv_split_views(torch.from_numpy(want).view(nb, 2, bs, H, fd), H, hs, Lg)
    for side in (0, 1):
        assert_same(host(dv[side].contiguous()), dh[side].contiguous().numpy(), f"data view side {side}")
        assert_same(host(sv[side].view(torch.uint8).contiguous()), sh[side].view(torch.uint8).contiguous().numpy(),
                    f"scale view side {side}")


def test_side_stream_and_graph_replay(g, orc):
    """Calls enqueued on a side stream (default priority) and a write +
    gather pair captured in a HIP graph give the oracle's bytes; the graph is
    replayed several times with eager work in between and every replay is
    checked (the kernels allocate nothing and issue no memset)."""
    w, g_tok, _ = synth.tiny_round_trip()
    want = np.full(8 * 64 * NV, 0xA5, np.uint8)
    orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, want, w.slot_mapping, 8, 64)
    rows = orc.gather_nvfp4_ds_mla(want, g_tok.total_tokens, g_tok.block_table, g_tok.workspace_starts,
                                   g_tok.seq_starts, 8, 64)
    kv, pe, sl = dev(w.kv_c), dev(w.k_pe), dev(w.slot_mapping)
    bt, ws, ss = dev(g_tok.block_table), dev(g_tok.workspace_starts), dev(g_tok.seq_starts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    cache = filled_cache((8, 64, NV), 0xA5)
    dst = torch.zeros((g_tok.total_tokens, 576), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(side):
        g.cache_write_nvfp4_ds_mla(kv, pe, cache, sl)
        g.cache_gather_upconvert_nvfp4_ds_mla(cache, dst, bt, ws, ss)
    side.synchronize()
    assert_same(host(cache).reshape(-1), want, "side-stream write")
    assert_same(host(dst), rows, "side-stream gather")

    cache2 = filled_cache((8, 64, NV), 0xA5)
    dst2 = torch.zeros_like(dst)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            g.cache_write_nvfp4_ds_mla(kv, pe, cache2, sl)
            g.cache_gather_upconvert_nvfp4_ds_mla(cache2, dst2, bt, ws, ss)
    torch.cuda.synchronize()
    for rep in range(4):
        cache2.fill_(0xA5)                               # eager work between replays
        dst2.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same(host(cache2).reshape(-1), want, f"graph replay {rep}: write")
        assert_same(host(dst2), rows, f"graph replay {rep}: gather")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_cache_offsets_beyond_4gib(g, orc, fmt):
    """A cache of more than 5 GiB: tokens written into its last four blocks
    (entry offsets above 2^32, so the kernels' 64-bit address arithmetic is
    exercised) and gathered back from there by two requests, against the
    oracle on a compact cache of just those four blocks; blocks below stay
    untouched."""
    eb, gwrite, ggather = _ds_pair(fmt)
    owrite, ogather = _orc_ds(orc, fmt)
    bs = 64
    nb = (5 << 30) // (bs * eb) + 1
    hi = nb - 4
    assert hi * bs * eb > (1 << 32)
    rng = np.random.default_rng(71)
    T = 4 * bs
    kv_c = synth.bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    k_pe = synth.bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    local = rng.permutation(T).astype(np.int64)
    local[::17] = -1
    compact = np.full(4 * bs * eb, 0xA5, np.uint8)
    owrite(kv_c, k_pe, compact, local, 4, bs)
    slots = np.where(local >= 0, local + hi * bs, -1)
    print(f"cache beyond 4 GiB: {fmt}, {nb} blocks, {nb * bs * eb / 2**30:.2f} GiB", flush=True)
    cache = torch.full((nb, bs, eb), 0xA5, dtype=torch.uint8, device="cuda")
    gwrite(dev(kv_c), dev(k_pe), cache, dev(slots))
    torch.cuda.synchronize()
    assert_same(host(cache[hi:]).reshape(-1), compact, f"{fmt} entries above 4 GiB")
    assert_same(host(cache[hi - 2:hi]).reshape(-1), np.full(2 * bs * eb, 0xA5, np.uint8), "blocks below")

    bt_local = np.array([[2, 0, 3, 1], [1, 3, -1, -1]], np.int32)
    ss = np.array([3, 0], np.int32)
    rows = np.array([4 * bs - 5, 2 * bs], np.int64) - ss
    ws = np.array([0, rows[0]], np.int32)
    total = int(rows.sum())
    want = ogather(compact, total, bt_local, ws, ss, 4, bs)
    bt = np.where(bt_local >= 0, bt_local + hi, -1).astype(np.int32)
    dst = torch.zeros((total, 576), dtype=torch.bfloat16, device="cuda")
    ggather(cache, dst, dev(bt), dev(ws), dev(ss))
    torch.cuda.synchronize()
    assert_same(host(dst), want, f"{fmt} gather from above 4 GiB")
    del cache


def test_perhead_cache_offsets_beyond_4gib(g, orc):
    """The per-head pair on a cache of more than 5 GiB (H = 8, head size 128,
    blocks of 16): tokens written into the last four blocks and gathered back
    one request per token, against the oracle on those four blocks alone."""
    H, hs, bs = 8, 128, 16
    fd = hs // 2 + hs // 16
    L = orc.kv_layout_split(bs, H, hs)
    nb = (5 << 30) // L.block_stride + 1
    hi = nb - 4
    assert hi * L.block_stride > (1 << 32)
    rng = np.random.default_rng(72)
    T = 4 * bs
    key = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * np.float32(3))
    value = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32))
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    local = rng.permutation(T).astype(np.int64)
    local[::13] = -1
    compact = np.full(4 * L.block_stride, 0xA5, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, compact, local, 4, bs, L, ks, vs)
    slots = np.where(local >= 0, local + hi * bs, -1)
    print(f"per-head cache beyond 4 GiB: {nb} blocks, {nb * L.block_stride / 2**30:.2f} GiB", flush=True)
    cache = torch.full((nb, 2, bs, H, fd), 0xA5, dtype=torch.uint8, device="cuda")
    ks_d = torch.tensor([ks], dtype=torch.float32, device="cuda")
    vs_d = torch.tensor([vs], dtype=torch.float32, device="cuda")
    g.reshape_and_cache_nvfp4(dev(key), dev(value), cache, dev(slots), ks_d, vs_d)
    torch.cuda.synchronize()
    assert_same(host(cache[hi:]).reshape(-1), compact, "per-head entries above 4 GiB")
    assert_same(host(cache[hi - 1]).reshape(-1), np.full(L.block_stride, 0xA5, np.uint8), "block below")

    gl = synth.per_token_gather("kv-high", local, 4, bs)
    ok, ov = orc.gather_upconvert_nvfp4_kv(compact, gl.total_tokens, gl.block_table, gl.workspace_starts,
                                           gl.seq_starts, H, hs, 4, bs, L, ks, vs)
    bt = (gl.block_table + hi).astype(np.int32)
    ko = torch.zeros((gl.total_tokens, H, hs), dtype=torch.bfloat16, device="cuda")
    vo = torch.zeros((gl.total_tokens, H, hs), dtype=torch.bfloat16, device="cuda")
    g.gather_upconvert_nvfp4_kv(cache, ko, vo, dev(bt), dev(gl.workspace_starts), ks_d, vs_d,
                                seq_starts=dev(gl.seq_starts))
    torch.cuda.synchronize()
    assert_same(host(ko), ok, "per-head K from above 4 GiB")
    assert_same(host(vo), ov, "per-head V from above 4 GiB")
    del cache


def _random_ds_case(rng):
    """One seeded random DS-MLA case: geometry, strides, padding and gather
    metadata drawn from ranges that cross the kernels' internal limits (tile
    of 16, one wave of 64 requests, power-of-two and generic block sizes)."""
    bs = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 128]))
    nb = int(rng.integers(1, 41))
    T = int(rng.integers(0, min(nb * bs, 700) + 1))
    pad = int(rng.integers(0, T // 3 + 1))
    ek, bk = int(rng.choice([0, 1, 3])), int(rng.choice([0, 2]))
    xk = int(rng.choice([0, 2]))
    B = int(rng.choice([1, 5, 63, 64, 65, 70]))
    maxb = int(rng.integers(1, 9))
    return dict(bs=bs, nb=nb, T=T, pad=pad, ek=ek, bk=bk, xk=xk, B=B, maxb=maxb,
                dst_extra=int(rng.choice([0, 8])), seed=int(rng.integers(1 << 30)))


def _extra_sweep_seeds():
    """GCACHE_SWEEP_SEEDS=N adds N more master seeds to each randomized sweep
    (0 by default; 150 ran bit-exact: 28,800 DS-MLA and 7,200 per-head
    cases on top of the default ones)."""
    return range(int(os.environ.get("GCACHE_SWEEP_SEEDS", "0")))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_randomized_ds_sweep(g, orc, fmt):
    """96 seeded random cases per format: block sizes 1..128 (power-of-two
    and generic division), 0..700 tokens with random padding, padded entry
    and block strides, strided inputs, 1..70 requests (both request searches)
    with random lengths, empty requests, seq_starts and shared blocks, and a
    wider dst row -- every cache byte and every output bit against the
    oracle."""
    seeds = [4242 if fmt == "nvfp4" else 4343]
    seeds += [100000 + 2 * k + (fmt == "fp8") for k in _extra_sweep_seeds()]
    for seed in seeds:
        _ds_sweep(g, orc, fmt, seed)


def _ds_sweep(g, orc, fmt, master_seed):
    eb = NV if fmt == "nvfp4" else F8
    master = np.random.default_rng(master_seed)
    for n in range(96):
        c = _random_ds_case(master)
        print(f"random DS case {fmt} master {master_seed} #{n}: {c}", flush=True)
        rng = np.random.default_rng(c["seed"])
        bs, nb, T = c["bs"], c["nb"], c["T"]
        estr = eb + 16 * c["ek"]
        bstr = bs * estr + 16 * c["bk"]
        width = 584 + 8 * c["xk"]
        buf = synth.bf16_bits(rng.standard_normal((T, width), dtype=np.float32)
                              * np.exp(rng.standard_normal((T, 1), dtype=np.float32)))
        kv_c, k_pe = buf[:, :512], buf[:, width - 64:]
        slots = synth.padded_slots(rng, nb * bs, T, c["pad"])
        if T:
            bdev = dev(buf)
            want, flat = run_ds_write(orc, fmt, kv_c, k_pe, slots, nb, bs, bstr, estr,
                                      kv_dev=bdev[:, :512], pe_dev=bdev[:, width - 64:])
        else:                           # nothing written: gather from an all-sentinel cache
            want, flat = np.full(nb * bstr, 0xA5, np.uint8), filled_cache((nb * bstr,), 0xA5)
        B, maxb = c["B"], c["maxb"]
        L = rng.integers(0, maxb * bs + 1, size=B)
        L[rng.random(B) < 0.15] = 0
        s = np.array([rng.integers(0, l + 1) for l in L], np.int64)
        rows = L - s
        bt = np.full((B, maxb), -1, np.int32)
        for b in range(B):
            nblk = -(-int(L[b]) // bs)
            bt[b, :nblk] = rng.integers(0, nb, size=nblk)      # blocks may repeat across requests
        ws = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int32)
        gcase = synth.GatherCase(f"random-{n}", bt, ws, s.astype(np.int32), int(rows.sum()), nb, bs, L)
        if gcase.total_tokens:
            run_ds_gather(orc, fmt, want, flat, gcase, nb, bs, bstr, estr, dst_stride=576 + c["dst_extra"])


def test_randomized_perhead_sweep(g, orc):
    """48 seeded random per-head cases: 1..9 heads, head sizes 16..256 (all
    multiples of 16), block sizes 1..32, the NHD or HND split layout or
    [data | scale] rows per (token, head) (staged kernels whenever a token's
    run is 16-byte aligned and at most 2048 bytes), 0..300 tokens with
    padding, gathered back per token -- every byte and bit."""
    for seed in [4444] + [200000 + k for k in _extra_sweep_seeds()]:
        _perhead_sweep(g, orc, seed)


def _perhead_sweep(g, orc, master_seed):
    master = np.random.default_rng(master_seed)
    for n in range(48):
        H = int(master.integers(1, 10))
        hs = int(master.choice([16, 32, 48, 64, 80, 128, 256]))
        bs = int(master.choice([1, 3, 8, 16, 32]))
        nb = int(master.integers(1, 25))
        T = int(master.integers(0, min(nb * bs, 300) + 1))
        pad = int(master.integers(0, T // 4 + 1))
        layout = str(master.choice(["nhd", "hnd", "rows"]))
        if layout == "rows" and hs % 128:
            hs = 128                    # [data | scale] rows keep 8-byte data alignment only at hs % 128 == 0
        seed = int(master.integers(1 << 30))
        print(f"random per-head case master {master_seed} #{n}: H={H} hs={hs} bs={bs} nb={nb} T={T} "
              f"pad={pad} layout={layout}",
              flush=True)
        rng = np.random.default_rng(seed)
        if T == 0:
            continue
        key, value, slots = _kv_case(rng, T, H, hs, nb, bs, pad)
        ks, vs = synth.global_scale(key), synth.global_scale(value)
        if layout == "rows":
            fd = hs // 2 + hs // 16
            kw = dict(data_offset=0, data_token_stride=H * fd, data_head_stride=fd, scale_offset=hs // 2,
                      scale_token_stride=H * fd, scale_head_stride=fd, side_stride=bs * H * fd,
                      block_stride=2 * bs * H * fd)
            L_orc, L_gpu = orc.KvLayout(**kw), g.NvFp4KvLayout(**kw)
        else:
            L_orc = orc.kv_layout_split(bs, H, hs, hnd=layout == "hnd")
            L_gpu = g.nvfp4_kv_split_layout(bs, H, hs, hnd=layout == "hnd")
        if any(v % 8 for v in (L_orc.data_offset, L_orc.data_token_stride, L_orc.data_head_stride,
                               L_orc.side_stride, L_orc.block_stride)):
            # e.g. a side of block_size * H * full_dim bytes that is not a multiple of 8: the
            # kernels' 8-byte code accesses would be misaligned, so the library refuses
            with pytest.raises(g.GcacheError) as e:
                run_kv(orc, g, key, value, slots, nb, bs, L_orc, L_gpu, ks, vs)
            assert e.value.status == -3
            continue
        run_kv(orc, g, key, value, slots, nb, bs, L_orc, L_gpu, ks, vs)


def test_binding_rejects_unsafe_arguments(g):
    """Arguments the kernels could not bound are refused before any launch:
    a block table whose rows are not contiguous, a batch larger than the
    metadata, and a per-head layout that reaches past the cache tensor."""
    cache = torch.zeros((4, 16, NV), dtype=torch.uint8, device="cuda")
    dst = torch.zeros((8, 576), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(2, dtype=torch.int32, device="cuda")
    wide = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        g.cache_gather_upconvert_nvfp4_ds_mla(cache, dst, wide[:, :3], ws)
    with pytest.raises(ValueError):
        g.cache_gather_upconvert_nvfp4_ds_mla(cache, dst, wide, ws, batch_size=3)
    H, hs, bs, nb = 2, 32, 4, 3
    fd = hs // 2 + hs // 16
    kv = torch.zeros((nb, 2, bs, H, fd), dtype=torch.uint8, device="cuda")
    L = g.nvfp4_kv_split_layout(bs, H, hs)
    L.block_stride += 64                        # the last block would run past the tensor
    key = torch.zeros((5, H, hs), dtype=torch.bfloat16, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        g.reshape_and_cache_nvfp4(key, key, kv, torch.zeros(5, dtype=torch.int64, device="cuda"), one, one,
                                  layout=L)
