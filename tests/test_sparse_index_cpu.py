"""Sparse index conversion in the oracle: hand-derived vectors, the length
check, and a NumPy brute force on random inputs."""
import numpy as np
import pytest

from conftest import load_golden


def test_hand_vectors(orc):
    g = load_golden("sparse_index_vectors.json")
    for case in g["cases"]:
        out = orc.convert_req_index(g["req_id"], g["token_indices"], g["block_table"], g["block_size"],
                                    case["num_blocks"])
        assert out.tolist() == case["out"]


def test_length_mismatch_is_rejected(orc):
    g = load_golden("sparse_index_vectors.json")
    with pytest.raises(orc.OracleError):
        orc.convert_req_index(g["req_id"] + [0], g["token_indices"], g["block_table"], g["block_size"], 10)
    with pytest.raises(orc.OracleError):
        orc.convert_req_index(g["req_id"][:-1], g["token_indices"], g["block_table"], g["block_size"], 10)


def brute(req_id, ti, bt, bs, nb):
    out = np.full(ti.shape, -1, np.int64)
    for t in range(ti.shape[0]):
        r = int(req_id[t])
        for k in range(ti.shape[1]):
            i = int(ti[t, k])
            if i < 0 or not 0 <= r < bt.shape[0] or i // bs >= bt.shape[1]:
                continue
            blk = int(bt[r, i // bs])
            if 0 <= blk < nb:
                out[t, k] = blk * bs + i % bs
    return out


def test_random_vs_brute_force(orc):
    rng = np.random.default_rng(17)
    for _ in range(20):
        B, mb, bs = int(rng.integers(1, 9)), int(rng.integers(1, 7)), int(rng.choice([1, 3, 16, 64]))
        nb = int(rng.integers(1, 50))
        bt = rng.integers(-2, nb + 3, size=(B, mb)).astype(np.int32)
        T, K = int(rng.integers(1, 30)), int(rng.integers(1, 40))
        req = rng.integers(-1, B + 2, size=T).astype(np.int32)
        ti = rng.integers(-3, mb * bs + 5, size=(T, K)).astype(np.int32)
        assert np.array_equal(orc.convert_req_index(req, ti, bt, bs, nb), brute(req, ti, bt, bs, nb))
