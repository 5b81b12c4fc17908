"""Chunked-context plan (the host metadata of a chunked prefill gather):
the oracle against hand-derived vectors and invariants, and the library's
host planner (gcache_context_chunk_plan / gcache_context_chunk, no device
needed) against the oracle."""
import numpy as np
import pytest

from conftest import load_golden


def test_oracle_chunk_plan_hand_vectors(orc):
    g = load_golden("context_chunk_vectors.json")
    for case in g["cases"]:
        c, chunks = orc.context_chunks(case["context_lens"], case["workspace_rows"], case["block_size"])
        assert c == case["chunk_rows"], case["name"]
        assert len(chunks) == case["num_chunks"], case["name"]
        for want in case["chunks"]:
            ss, ws, tot = chunks[want["chunk"]]
            assert ss.tolist() == want["seq_starts"], case["name"]
            assert ws.tolist() == want["workspace_starts"], case["name"]
            assert tot == want["total_rows"], case["name"]
    for bad in g["errors"]:
        with pytest.raises(orc.OracleError):
            orc.context_chunks(bad["context_lens"], bad["workspace_rows"], bad["block_size"])


def test_oracle_chunk_plan_invariants(orc):
    """Every context position of every request is gathered exactly once, in
    order; no chunk exceeds the workspace; the chunk size is the largest
    multiple of the block size that fits."""
    rng = np.random.default_rng(8)
    for _ in range(60):
        B = int(rng.integers(1, 12))
        bs = int(rng.choice([1, 16, 64]))
        lens = rng.integers(0, 3000, size=B).astype(np.int32)
        lens[rng.random(B) < 0.2] = 0
        wrows = int(rng.integers(B * bs, B * bs * 40 + 1))
        c, chunks = orc.context_chunks(lens, wrows, bs)
        assert c % bs == 0 and B * c <= wrows < B * (c + bs)
        seen = [[] for _ in range(B)]
        for ss, ws, tot in chunks:
            assert tot <= wrows
            rows = np.diff(np.concatenate([ws, [tot]]))
            for b in range(B):
                seen[b].extend(range(int(ss[b]), int(ss[b]) + int(rows[b])))
        for b in range(B):
            assert seen[b] == list(range(int(lens[b])))


def test_library_planner_matches_oracle(orc):
    import gather_concat_cache_amd as gc
    rng = np.random.default_rng(9)
    for _ in range(80):
        B = int(rng.integers(1, 70))
        bs = int(rng.choice([1, 8, 16, 64]))
        lens = rng.integers(0, 5000, size=B).astype(np.int32)
        wrows = int(rng.integers(B * bs, B * bs * 30 + 1))
        c1, ch1 = gc.context_chunks(lens, wrows, bs)
        c2, ch2 = orc.context_chunks(lens, wrows, bs)
        assert c1 == c2 and len(ch1) == len(ch2)
        for (a, b, t), (x, y, u) in zip(ch1, ch2):
            assert np.array_equal(a, x) and np.array_equal(b, y) and t == u
    for bad in load_golden("context_chunk_vectors.json")["errors"]:
        with pytest.raises(gc.GcacheError):
            gc.context_chunks(bad["context_lens"], bad["workspace_rows"], bad["block_size"])
