"""Host-side logic of bench.py, on the CPU: the request shards the all-cores
oracle baseline runs (contiguous, covering exactly the sampled rows, cut at
request boundaries), the sharded oracle gather against the one-call result,
and the mapping from rocprofv3 kernel names (templated write kernels
included) to op names."""
import numpy as np
import pytest

import bench


def _ws(rng, batch, empty_frac=0.2, max_len=300):
    lens = rng.integers(1, max_len, size=batch)
    lens[rng.random(batch) < empty_frac] = 0
    ws = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    return ws, int(lens.sum())


@pytest.mark.parametrize("seed", range(6))
def test_request_shards_cover_rows(seed):
    rng = np.random.default_rng(seed)
    ws, total = _ws(rng, int(rng.integers(1, 80)))
    if total == 0:
        return
    for n in {1, total // 3 + 1, total}:
        for parts in (1, 3, 16, 200):
            sh = bench._request_shards(ws, total, n, parts)
            assert sh[0][2] == 0 and sh[-1][3] == n
            for (b0, b1, r0, r1), nxt in zip(sh, sh[1:] + [None]):
                assert 0 <= b0 < b1 <= len(ws) and r0 == ws[b0] and r0 < r1 <= n
                if nxt is not None:
                    assert nxt[0] == b1 and nxt[2] == r1
            assert len(sh) <= max(parts, 1) + 1 or parts >= len(ws)


def test_sharded_oracle_gather_matches_one_call(orc):
    import synth
    rng = np.random.default_rng(11)
    nb, bs = 16, 8
    w = synth.random_write(11, 100, nb, bs, 5)
    cache = np.zeros(nb * bs * 352, np.uint8)
    orc.write_nvfp4_ds_mla(w.kv_c, w.k_pe, cache, w.slot_mapping, nb, bs)
    batch = 9
    lens = rng.integers(0, 20, size=batch)
    ws = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total = int(lens.sum())
    ss = rng.integers(0, 5, size=batch).astype(np.int32)
    bt = rng.integers(0, nb, size=(batch, 4)).astype(np.int32)
    ref = orc.gather_nvfp4_ds_mla(cache, total, bt, ws, ss, nb, bs)
    for parts in (1, 2, 4, 16):
        dst = np.zeros((total, 576), np.uint16)
        for b0, b1, r0, r1 in bench._request_shards(ws, total, total, parts):
            sub = (ws[b0:b1] - ws[b0]).astype(np.int32)
            orc.gather_nvfp4_ds_mla(cache, r1 - r0, bt[b0:b1], sub, ss[b0:b1], nb, bs, dst=dst[r0:r1])
        assert np.array_equal(dst, ref), parts


def test_kernel_names_map_to_ops():
    assert bench.kernel_op("void gcache::k_write_nvfp4_ds_mla<1, 2>(gcache::DsMlaWriteParams, long)") == \
        "nvfp4_ds_mla_write"
    assert bench.kernel_op("void gcache::k_write_fp8_ds_mla<2, 4>(gcache::DsMlaWriteParams, long)") == \
        "fp8_ds_mla_write"
    assert bench.kernel_op("void gcache::k_gather_ds_mla<true>(gcache::DsMlaGatherParams, long)") == \
        "nvfp4_ds_mla_gather"
    assert bench.kernel_op("void gcache::k_gather_ds_mla<false>(gcache::DsMlaGatherParams, long)") == \
        "fp8_ds_mla_gather"
    for staged in ("true", "false"):          # the staged and the direct per-head kernels are one op each
        assert bench.kernel_op(f"void gcache::k_gather_nvfp4_kv<{staged}>(gcache::KvGatherParams, long)") == \
            "nvfp4_kv_gather"
        assert bench.kernel_op(f"void gcache::k_reshape_and_cache_nvfp4<{staged}>(gcache::KvWriteParams, long)") == \
            "nvfp4_kv_write"
    assert bench.kernel_op("gcache::k_gather_bf16(gcache::DsMlaGatherParams, long)") is None
    assert bench.kernel_op("void gcache::k_convert_req_index<true>(gcache::SparseIndexParams, long)") is None


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and a
    message, before touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
