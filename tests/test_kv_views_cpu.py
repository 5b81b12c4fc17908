"""Per-head split layouts and views: the oracle's and the library's NHD/HND
layout functions against hand-derived values, and the binding's split views
(torch views over a CPU cache written by the oracle) against the NumPy
brute-force quantizer, head by head."""
import numpy as np
import pytest
import torch

import brute
import synth
from conftest import load_golden

FIELDS = ("data_offset", "data_token_stride", "data_head_stride", "scale_offset", "scale_token_stride",
          "scale_head_stride", "side_stride", "block_stride")


def test_split_layout_hand_values(orc):
    import gather_concat_cache_amd as gc
    g = load_golden("kv_split_layouts.json")
    for order in ("nhd", "hnd"):
        a = orc.kv_layout_split(g["block_size"], g["num_heads"], g["head_size"], hnd=order == "hnd")
        b = gc.nvfp4_kv_split_layout(g["block_size"], g["num_heads"], g["head_size"], hnd=order == "hnd")
        for f in FIELDS:
            assert getattr(a, f) == g[order][f], (order, f)
            assert getattr(b, f) == g[order][f], (order, f)


@pytest.mark.parametrize("order", ["nhd", "hnd"])
def test_split_views_match_brute_force(orc, order):
    import gather_concat_cache_amd as gc
    rng = np.random.default_rng(29)
    T, H, hs, nb, bs = 30, 3, 64, 6, 8
    key = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32))
    value = synth.bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * np.float32(3))
    ks, vs = synth.global_scale(key), synth.global_scale(value)
    L = orc.kv_layout_split(bs, H, hs, hnd=order == "hnd")
    slots = synth.padded_slots(rng, nb * bs, T, 3)
    fd = hs // 2 + hs // 16
    cache = np.zeros(nb * 2 * bs * H * fd, np.uint8)
    orc.reshape_and_cache_nvfp4(key, value, cache, slots, nb, bs, L, ks, vs)
    t5 = torch.from_numpy(cache).view(nb, 2, bs, H, fd)
    data, scale = gc.nvfp4_kv_split_views(t5, H, hs, gc.nvfp4_kv_split_layout(bs, H, hs, hnd=order == "hnd"))
    assert data[0].shape == (nb, bs, H, hs // 2) and scale[0].dtype == torch.float8_e4m3fn
    for side, (x, gs) in enumerate(((key, ks), (value, vs))):
        d, sc = brute.kv_quantize(x, gs)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            assert np.array_equal(data[side][s // bs, s % bs].numpy(), d[t])
            assert np.array_equal(scale[side][s // bs, s % bs].view(torch.uint8).numpy(), sc[t])
