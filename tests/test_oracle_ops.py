"""Pins of the oracle's six operations against things other than itself.

* closed forms from the pages (entry sizes, full_dim and its split);
* hand-derived vectors (tests/golden/*_vectors.json);
* the pages' own write-test tolerances (1-ulp scale byte against a reference
  scale computed with torch's float8_e4m3fn cast, |deq - x| <= 1.5 * scale,
  RoPE |deq - x| <= |x| / 8 + 2^-9) and the tighter half-step bounds;
* NumPy brute force (tests/brute.py) on small inputs, every byte and bit;
* invariants: padding and untouched bytes keep their sentinel, the gather walk
  agrees with slot ids encoded into RoPE values, the per-head write with
  gs = 1 on a 512-wide head reproduces the DS-MLA NoPE bytes;
* error handling of invalid inputs.
"""
import numpy as np
import pytest
import torch

import brute
import synth
from conftest import load_golden
from synth import bf16_bits, bf16_to_f32

NV, F8 = 352, 656


def _block_row(values):
    row = np.zeros((1, 512), np.float32)
    row[0, :len(values)] = values
    return bf16_bits(row)


def _write_one(orc, kv_c, k_pe=None, fmt="nvfp4"):
    k_pe = bf16_bits(np.zeros((kv_c.shape[0], 64), np.float32)) if k_pe is None else k_pe
    eb = NV if fmt == "nvfp4" else F8
    cache = np.full(eb * kv_c.shape[0], 0xA5, np.uint8)
    slots = np.arange(kv_c.shape[0], dtype=np.int64)
    fn = orc.write_nvfp4_ds_mla if fmt == "nvfp4" else orc.write_fp8_ds_mla
    fn(kv_c, k_pe, cache, slots, 1, kv_c.shape[0])
    return cache.reshape(-1, eb)


# ---------------------------------------------------------------------------
def test_closed_forms(orc):
    g = load_golden("formats.json")
    assert orc.nvfp4_ds_mla_entry_bytes() == g["nvfp4_ds_mla_entry_bytes"] == sum(g["nvfp4_ds_mla_parts"].values())
    assert orc.fp8_ds_mla_entry_bytes() == g["fp8_ds_mla_entry_bytes"] == 512 + 16 + 128
    for hs, fd in g["full_dim"].items():
        assert orc.nvfp4_full_dim(int(hs)) == fd
    for hs, dd in g["data_dim"].items():
        fd = orc.nvfp4_full_dim(int(hs))
        assert fd * 8 // 9 == dd == int(hs) // 2
        assert fd - dd == g["scale_dim"][hs] == int(hs) // 16
    L = orc.kv_layout_split(16, 8, 128)
    assert L.block_stride == 2 * 16 * 8 * 72 and L.side_stride == 16 * 8 * 72
    assert L.scale_offset == 16 * 8 * 64 and L.data_head_stride == 64 and L.scale_head_stride == 8


def test_nvfp4_block_hand_vectors(orc):
    g = load_golden("nvfp4_ds_mla_vectors.json")
    for blk in g["blocks"]:
        e = _write_one(orc, _block_row(blk["values"]))[0]
        assert e[320] == int(blk["scale_byte"], 16), blk["name"]
        assert e[:8].tobytes().hex() == blk["packed"], blk["name"]
        assert np.all(e[321:352] == 0) and np.all(e[8:256] == 0)     # other blocks are zero
        d = orc.gather_nvfp4_ds_mla(e.copy(), 1, np.zeros((1, 1), np.int32), np.zeros(1, np.int32),
                                    None, 1, 1)
        got = bf16_to_f32(d[0, :16])
        want = np.array(blk["dequant"], np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), blk["name"]
    r = g["rope"]
    k_pe = np.zeros((1, 64), np.float32)
    k_pe[0, :len(r["values"])] = r["values"]
    e = _write_one(orc, _block_row([]), bf16_bits(k_pe))[0]
    assert [f"{c:#04x}" for c in e[256:256 + len(r["codes"])]] == r["codes"]


def test_fp8_hand_vectors(orc):
    g = load_golden("fp8_ds_mla_vectors.json")
    row = np.zeros((1, 512), np.float32)
    for gi, grp in enumerate(g["groups"]):
        row[0, 128 * gi:128 * gi + len(grp["values_head"])] = grp["values_head"]
    k_pe = np.zeros((1, 64), np.uint16)
    k_pe[0, :2] = [int(b, 16) for b in g["rope_bf16_bits"]]
    e = _write_one(orc, bf16_bits(row), k_pe, fmt="fp8")[0]
    for gi, grp in enumerate(g["groups"]):
        n = len(grp["codes_head"])
        assert [f"{c:#04x}" for c in e[128 * gi:128 * gi + n]] == grp["codes_head"], grp["name"]
        assert np.all(e[128 * gi + n:128 * (gi + 1)] == 0), grp["name"]
        assert e[512 + 4 * gi:516 + 4 * gi].tobytes().hex() == grp["scale_le"], grp["name"]
    assert e[528:532].tobytes().hex() == g["rope_bytes"]
    d = orc.gather_fp8_ds_mla(e.copy(), 1, np.zeros((1, 1), np.int32), np.zeros(1, np.int32), None, 1, 1)
    grp = g["groups"][3]
    assert list(bf16_to_f32(d[0, 384:386])) == grp["dequant_head"]
    assert list(d[0, 512:514]) == [0x3F80, 0xC020]


def golden_gs(h):
    """A fixture's per-tensor scale: exact binary32 bits when given, else a
    value that is exact in binary32."""
    if "gs_bits" in h:
        return float(np.array(int(h["gs_bits"], 16), np.uint32).view(np.float32))
    return float(np.float32(h["gs"]))


def test_perhead_hand_vectors(orc):
    """Per-head blocks through the oracle's write and gather.  The last two
    heads take a per-tensor scale that is not a power of two: one fixes the
    order of the scale computation ((amax / 6) / gs), the other the two
    roundings of the dequant (binary32, then bf16)."""
    g = load_golden("perhead_vectors.json")
    for h in g["heads"]:
        gs = golden_gs(h)
        key = bf16_bits(np.array(h["values"], np.float32).reshape(1, 1, 16))
        L = orc.kv_layout_split(1, 1, 16)
        cache = np.full(2 * 9, 0xA5, np.uint8)
        orc.reshape_and_cache_nvfp4(key, key, cache, np.zeros(1, np.int64), 1, 1, L, gs, gs)
        for side in (0, 1):
            assert cache[9 * side:9 * side + 8].tobytes().hex() == h["data"], h["name"]
            assert cache[9 * side + 8] == int(h["scale_byte"], 16), h["name"]
        k, v = orc.gather_upconvert_nvfp4_kv(cache, 1, np.zeros((1, 1), np.int32), np.zeros(1, np.int32),
                                             None, 1, 16, 1, 1, L, gs, gs)
        assert np.array_equal(v, k), h["name"]
        if "dequant_bf16" in h:
            assert np.all(k == int(h["dequant_bf16"], 16)), h["name"]
        elif "dequant_bits" in h:
            want = np.array([int(b, 16) for b in h["dequant_bits"]], np.uint16)
            assert np.array_equal(k[0, 0], want), h["name"]
        else:
            want = np.array(h["dequant"], np.float32)
            assert np.array_equal(bf16_to_f32(k[0, 0]).view(np.uint32), want.view(np.uint32)), h["name"]


def fp8_gather_rounding_entry(case):
    """The hand-built fp8_ds_mla entry of the gather rounding case: its codes
    lead group 0, whose scale has the given bits; everything else is zero."""
    e = np.zeros(F8, np.uint8)
    e[:len(case["codes"])] = [int(c, 16) for c in case["codes"]]
    e[512:516] = np.array([int(case["scale_bits"], 16)], "<u4").view(np.uint8)
    return e


def test_fp8_rounding_order_hand_vectors(orc):
    """fp8_ds_mla with a scale that is not a power of two: the write
    multiplies by the binary32 reciprocal of the scale (not a division), and
    the gather rounds the binary32 product to bf16 (two roundings)."""
    g = load_golden("fp8_ds_mla_vectors.json")
    w = g["write_rounding"]
    row = np.zeros((1, 512), np.float32)
    row[0, :len(w["values_head"])] = w["values_head"]
    e = _write_one(orc, bf16_bits(row), fmt="fp8")[0]
    assert [f"{c:#04x}" for c in e[:len(w["codes_head"])]] == w["codes_head"]
    assert e[512:516].tobytes().hex() == w["scale_le"]
    d = orc.gather_fp8_ds_mla(e.copy(), 1, np.zeros((1, 1), np.int32), np.zeros(1, np.int32), None, 1, 1)
    assert list(bf16_to_f32(d[0, :len(w["dequant_head"])])) == w["dequant_head"]
    r = g["gather_rounding"]
    d = orc.gather_fp8_ds_mla(fp8_gather_rounding_entry(r), 1, np.zeros((1, 1), np.int32),
                              np.zeros(1, np.int32), None, 1, 1)
    assert [f"{b:#06x}" for b in d[0, :len(r["codes"])]] == r["dequant_bf16"]


def test_gather_walk_hand_vectors(orc):
    for c in load_golden("gather_walk_vectors.json")["cases"]:
        bt = np.array(c["block_table"], np.int32)
        ws = np.array(c["workspace_starts"], np.int32)
        ss = None if c["seq_starts"] is None else np.array(c["seq_starts"], np.int32)
        blk, off = orc.gather_walk(c["total_tokens"], bt, ws, ss, c["num_blocks"], c["block_size"])
        assert blk.tolist() == c["blocks"] and off.tolist() == c["offsets"], c["name"]


# ---------------------------------------------------------------------------
def _page_tolerance_checks(entries, kv_c, k_pe):
    """The write test of the PR51724 digest (Key source excerpts), restated:
    scale bytes within one e4m3 ulp of a reference from amax / 6.0 (computed
    here with torch's float8_e4m3fn cast), NoPE |deq - x| <= 1.5 * scale,
    RoPE |deq - x| <= |x| * 2^-3 + 2^-9."""
    x = bf16_to_f32(kv_c).reshape(-1, 32, 16)
    amax = np.abs(x).max(axis=2)
    ref = torch.from_numpy((amax / np.float32(6.0)).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy().astype(np.int16)
    sf = entries[:, 320:352]
    assert np.all(np.abs(sf.astype(np.int16) - ref) <= 1)
    s = brute.e4m3_value(sf)
    nib = np.stack([entries[:, :256] & 0xF, entries[:, :256] >> 4], axis=2).reshape(-1, 32, 16)
    deq = brute.e2m1_value(nib) * s[:, :, None]
    assert np.all(np.abs(deq - x) <= 1.5 * s[:, :, None])
    r = bf16_to_f32(k_pe).astype(np.float64)
    rd = brute.e4m3_value(entries[:, 256:320])
    assert np.all(np.abs(rd - r) <= np.abs(r) * 2.0 ** -3 + 2.0 ** -9)
    return x, s, deq


def _tight_bounds(x, s, deq):
    """Half-step bound where the scale is normal and unsaturated:
    |x - deq| <= halfstep(|code|) * scale (0.25, 0.5, 1 below 2, 4, 6)."""
    amax6 = np.abs(x).max(axis=2) / 6.0
    ok = (amax6 >= 2.0 ** -6) & (amax6 <= 448)
    q = np.abs(deq) / np.where(s == 0, 1, s)[:, :, None]
    half = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    err = np.abs(x - deq)
    bound = half * s[:, :, None] * (1 + 2.0 ** -20)
    assert np.all((err <= bound)[ok])
    return int((~ok).sum())


def test_page_tolerances_tiny_and_decode_workloads(orc):
    w1, _, _ = synth.tiny_round_trip()
    w2 = synth.decode_batch_write()
    for w in (w1, w2):
        valid = w.slot_mapping >= 0
        cache = np.full(w.num_blocks * w.block_size * NV, 0xA5, np.uint8)
        orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache, w.slot_mapping, w.num_blocks, w.block_size)
        ent = cache.reshape(-1, NV)[w.slot_mapping[valid]]
        x, s, deq = _page_tolerance_checks(ent, w.kv_c[valid], w.k_pe[valid])
        excluded = _tight_bounds(x, s, deq)
        if w is w2:
            assert excluded > 0          # the x50 outliers of lognormal tokens saturate some scales


def test_nvfp4_write_and_gathers_vs_brute_force_tiny(orc):
    w, g_tok, g_all = synth.tiny_round_trip()
    cache = np.full(w.num_blocks * w.block_size * NV, 0xA5, np.uint8)
    orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache, w.slot_mapping, w.num_blocks, w.block_size)
    want = np.full_like(cache, 0xA5)
    brute.scatter(want, brute.nvfp4_ds_mla_entries(w.kv_c, w.k_pe), w.slot_mapping, 64, 64 * NV, NV)
    assert np.array_equal(cache, want)                       # every byte, padding included
    for g in (g_tok, g_all):
        d = orc.gather_nvfp4_ds_mla(cache, g.total_tokens, g.block_table, g.workspace_starts,
                                    g.seq_starts, g.num_blocks, g.block_size)
        blk, off = brute.walk(g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, 64)
        rows = brute.nvfp4_rows(brute.read_entries(cache, blk, off, 64 * NV, NV, NV))
        assert np.array_equal(d, rows), g.name


def test_strided_inputs_and_padded_entries_vs_brute_force(orc):
    """kv_c / k_pe as slices of one [T, 576] tensor, entry_stride 384 > 352,
    block_stride with a gap: the oracle addresses everything through strides."""
    rng = np.random.default_rng(5)
    T, nb, bs, es, bstr = 50, 6, 16, 384, 16 * 384 + 128
    full = bf16_bits(rng.standard_normal((T, 576), dtype=np.float32) * np.float32(3))
    kv_c, k_pe = full[:, :512], full[:, 512:]
    slots = synth.padded_slots(rng, nb * bs, T, 5)
    cache = np.full(nb * bstr, 0x5A, np.uint8)
    orc.write_nvfp4_ds_mla(kv_c, k_pe, cache, slots, nb, bs, bstr, es)    # strided row views
    want = np.full_like(cache, 0x5A)
    brute.scatter(want, brute.nvfp4_ds_mla_entries(np.ascontiguousarray(kv_c), np.ascontiguousarray(k_pe)),
                  slots, bs, bstr, es)
    assert np.array_equal(cache, want)
    g = synth.per_token_gather("g", slots, nb, bs)
    dst = np.full((g.total_tokens, 600), 0x1234, np.uint16)           # dst_stride 600 > 576
    orc.gather_nvfp4_ds_mla(cache, g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts,
                            nb, bs, bstr, es, dst=dst)
    blk, off = brute.walk(g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, bs)
    assert np.array_equal(dst[:, :576], brute.nvfp4_rows(brute.read_entries(cache, blk, off, bstr, es, NV)))
    assert np.all(dst[:, 576:] == 0x1234)                              # beyond the row: untouched


def test_fp8_write_and_gather_vs_brute_force(orc):
    rng = np.random.default_rng(9)
    T, nb, bs = 96, 8, 16
    kv_c = bf16_bits(rng.standard_normal((T, 512), dtype=np.float32)
                     * np.exp(rng.standard_normal((T, 1), dtype=np.float32)))
    kv_c[3, :128] = 0                                                  # a zero group
    k_pe = bf16_bits(rng.standard_normal((T, 64), dtype=np.float32))
    slots = synth.padded_slots(rng, nb * bs, T, 7)
    cache = np.full(nb * bs * F8, 0xA5, np.uint8)
    orc.write_fp8_ds_mla(kv_c, k_pe, cache, slots, nb, bs)
    want = np.full_like(cache, 0xA5)
    brute.scatter(want, brute.fp8_ds_mla_entries(kv_c, k_pe), slots, bs, bs * F8, F8)
    assert np.array_equal(cache, want)
    g = synth.prefill_gather(rng, "g", 4, 1, 32, nb, bs, 2)
    d = orc.gather_fp8_ds_mla(cache, g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, nb, bs)
    blk, off = brute.walk(g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, bs)
    assert np.array_equal(d, brute.fp8_rows(brute.read_entries(cache, blk, off, bs * F8, F8, F8)))
    # error bound of the fp8 round trip: |x - deq| <= half an e4m3 step of |x|
    valid = slots >= 0
    dv = orc.gather_fp8_ds_mla(cache, int(valid.sum()), (slots[valid] // bs).astype(np.int32)[:, None],
                               np.arange(valid.sum(), dtype=np.int32), (slots[valid] % bs).astype(np.int32),
                               nb, bs)
    x = bf16_to_f32(kv_c[valid]).astype(np.float64)
    deq = bf16_to_f32(dv[:, :512]).astype(np.float64)
    sc = np.repeat(np.abs(x).reshape(-1, 4, 128).max(axis=2) / 448, 128, axis=1)
    assert np.all(np.abs(x - deq) <= np.abs(x) * 2.0 ** -4 + sc * 2.0 ** -9 + np.abs(x) * 2.0 ** -8)
    assert np.array_equal(dv[:, 512:], k_pe[valid])                    # RoPE copied bit for bit


@pytest.mark.parametrize("layout", ["split", "interleaved"])
def test_perhead_write_and_gather_vs_brute_force(orc, layout):
    rng = np.random.default_rng(13)
    T, H, hs, nb, bs = 40, 3, 32, 16, 4
    key = bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * rng.uniform(0.1, 10, (1, H, 1)).astype(np.float32))
    value = bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * np.float32(0.01))
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    fd = hs // 2 + hs // 16
    if layout == "split":
        L = orc.kv_layout_split(bs, H, hs)
    else:   # each (token, head) row is [data | scales]
        L = orc.KvLayout(data_offset=0, data_token_stride=H * fd, data_head_stride=fd,
                         scale_offset=hs // 2, scale_token_stride=H * fd, scale_head_stride=fd,
                         side_stride=bs * H * fd, block_stride=2 * bs * H * fd)
    slots = synth.padded_slots(rng, nb * bs, T, 4)
    cache = np.full(nb * 2 * bs * H * fd, 0xA5, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, cache, slots, nb, bs, L, ks, vs)
    want = np.full_like(cache, 0xA5)
    for side, (x, gs) in enumerate(((key, ks), (value, vs))):
        data, sc = brute.kv_quantize(x, gs)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            base = (s // bs) * L.block_stride + side * L.side_stride
            for h in range(H):
                a = base + L.data_offset + (s % bs) * L.data_token_stride + h * L.data_head_stride
                want[a:a + hs // 2] = data[t, h]
                a = base + L.scale_offset + (s % bs) * L.scale_token_stride + h * L.scale_head_stride
                want[a:a + hs // 16] = sc[t, h]
    assert np.array_equal(cache, want)
    g = synth.per_token_gather("g", slots, nb, bs)
    k, v = orc.gather_upconvert_nvfp4_kv(cache, g.total_tokens, g.block_table, g.workspace_starts,
                                         g.seq_starts, H, hs, nb, bs, L, ks, vs)
    valid = slots >= 0
    for out, x, gs in ((k, key, ks), (v, value, vs)):
        data, sc = brute.kv_quantize(x[valid], gs)
        assert np.array_equal(out, brute.kv_dequant(data, sc, gs))


def test_perhead_with_unit_scale_matches_ds_mla_nope(orc):
    """Special case: a 512-wide head with gs = 1 quantizes exactly like the
    DS-MLA NoPE part (same block rule, same nibble order, same scales)."""
    w, _, _ = synth.tiny_round_trip()
    T = 16
    kv_c, k_pe = w.kv_c[:T], w.k_pe[:T]
    ent = _write_one(orc, np.ascontiguousarray(kv_c), np.ascontiguousarray(k_pe))
    L = orc.kv_layout_split(T, 1, 512)
    cache = np.zeros(2 * T * 288, np.uint8)
    key = np.ascontiguousarray(kv_c.reshape(T, 1, 512))
    orc.reshape_and_cache_nvfp4(key, key, cache, np.arange(T, dtype=np.int64), 1, T, L, 1.0, 1.0)
    data = cache[:T * 256].reshape(T, 256)
    scales = cache[T * 256:T * 288].reshape(T, 32)
    assert np.array_equal(data, ent[:, :256]) and np.array_equal(scales, ent[:, 320:352])


def test_address_tags_pin_the_walk(orc):
    """Slot ids written as base-16 digits into five RoPE values (integers
    0..15 are exact in e4m3 and bf16) come back from the gather in the rows a
    linear-scan walk predicts: the walk is pinned without any quantization."""
    rng = np.random.default_rng(21)
    nb, bs = 64, 16
    T = nb * bs
    slots = np.arange(T, dtype=np.int64)
    digits = (slots[:, None] >> (4 * np.arange(5))[None, :]) & 15
    rope = np.zeros((T, 64), np.float32)
    rope[:, :5] = digits
    kv_c = bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    cache = np.zeros(nb * bs * NV, np.uint8)
    orc.write_nvfp4_ds_mla(kv_c, bf16_bits(rope), cache, slots, nb, bs)
    g = synth.prefill_gather(rng, "tags", 7, 3, 120, nb, bs, 8)
    d = orc.gather_nvfp4_ds_mla(cache, g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, nb, bs)
    got = (bf16_to_f32(d[:, 512:517]).astype(np.int64) << (4 * np.arange(5))[None, :]).sum(axis=1)
    blk, off = brute.walk(g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, bs)
    assert np.array_equal(got, blk * bs + off)


def test_bf16_comparator_gather_vs_brute_force(orc):
    """The BF16 comparator copies the 1152 entry bytes of the row that a
    linear-scan walk names, as 576 little-endian bf16 values: random cache
    bytes, padded entries, gaps between blocks, empty requests."""
    rng = np.random.default_rng(33)
    nb, bs = 12, 16
    estr = 1152 + 64
    bstr = bs * estr + 128
    cache = rng.integers(0, 256, size=nb * bstr, dtype=np.uint8)
    g = synth.prefill_gather(rng, "bf16", 5, 0, 40, nb, bs, 3)
    d = orc.gather_bf16(cache, g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, nb, bs,
                        bstr, estr)
    blk, off = brute.walk(g.total_tokens, g.block_table, g.workspace_starts, g.seq_starts, bs)
    want = np.stack([cache[b * bstr + o * estr: b * bstr + o * estr + 1152].view("<u2")
                     for b, o in zip(blk, off)]) if g.total_tokens else np.zeros((0, 576), np.uint16)
    assert np.array_equal(d, want)


def test_padding_and_untouched_bytes_keep_sentinels(orc):
    w = synth.decode_batch_write()
    for fill in (0xA5, 0x5A):
        for fmt, eb in (("nvfp4", NV), ("fp8", F8)):
            cache = np.full(w.num_blocks * w.block_size * eb, fill, np.uint8)
            fn = orc.write_nvfp4_ds_mla if fmt == "nvfp4" else orc.write_fp8_ds_mla
            fn(w.kv_c, w.k_pe, cache, w.slot_mapping, w.num_blocks, w.block_size)
            written = np.zeros(w.num_blocks * w.block_size, bool)
            written[w.slot_mapping[w.slot_mapping >= 0]] = True
            assert np.all(cache.reshape(-1, eb)[~written] == fill)


def test_invalid_inputs_are_rejected(orc):
    w, _, _ = synth.tiny_round_trip()
    cache = np.zeros(8 * 64 * NV, np.uint8)
    dup = w.slot_mapping.copy()
    dup[1] = dup[0] = 5
    with pytest.raises(orc.OracleError) as e:
        orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache, dup, 8, 64)
    assert e.value.status == -3 and not cache.any()
    bad = w.slot_mapping.copy()
    bad[0] = 512
    with pytest.raises(orc.OracleError) as e:
        orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache, bad, 8, 64)
    assert e.value.status == -2
    inf = w.kv_c.copy()
    inf[int(np.nonzero(w.slot_mapping >= 0)[0][0]), 7] = 0x7F80
    with pytest.raises(orc.OracleError) as e:
        orc.write_nvfp4_ds_mla(inf, w.k_pe, cache, w.slot_mapping, 8, 64)
    assert e.value.status == -4 and not cache.any()
    with pytest.raises(orc.OracleError) as e:
        orc.gather_walk(3, np.zeros((1, 1), np.int32), np.array([1], np.int32), None, 8, 64)
    assert e.value.status == -5
    with pytest.raises(orc.OracleError):
        orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache[:-1], w.slot_mapping, 8, 64)   # cache too small
