"""Seeded synthetic inputs for the paged KV-cache write and gather workloads.

This module only draws random numbers and lays out metadata (slot mappings,
block tables, workspace starts).  It holds none of the quantization or
dequantization arithmetic, so both the CPU oracle and the HIP library can
consume what it produces without sharing any of the method's code.

All draws use NumPy's PCG64 (``numpy.random.default_rng``).  Floating-point
values are drawn in float32 and rounded once, to nearest-even, to bf16; the
arrays returned hold raw bf16 bits as ``uint16``.  Workload shapes follow the
decode-batch and prefill shapes of the pages (DS-MLA: 512-wide NoPE latent +
64-wide RoPE, block size 64; per-head: 8 KV heads of size 128, block size 16).
"""
from dataclasses import dataclass, field

import numpy as np

NOPE, ROPE = 512, 64


def bf16_bits(x):
    """float32 array -> bf16 bits (uint16), round to nearest even.  Finite input only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b):
    """bf16 bits -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed, stream=None):
    return np.random.default_rng(seed if stream is None else [seed, stream])


def _normal_bf16(rng, shape):
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


CHUNK_ROWS = 8192


def normal_bf16_rows(seed, stream, rows, cols):
    """N(0,1) bf16 bits [rows, cols], drawn in chunks of CHUNK_ROWS rows;
    chunk c uses its own generator default_rng([seed, stream, c]), so the
    result does not depend on how many threads fill it."""
    import concurrent.futures as cf
    import os
    out = np.empty((rows, cols), np.uint16)
    nchunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def fill(c):
        lo, hi = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        x = np.random.default_rng([seed, stream, c]).standard_normal((hi - lo, cols), dtype=np.float32)
        u = x.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        np.right_shift(u, np.uint32(16), out=u)
        out[lo:hi] = u
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(fill, range(nchunks)))
    return out


def padded_slots(rng, num_slots, num_tokens, pad_count, sequential=False):
    """Distinct slots (random draw without replacement, or 0..T-1), with
    exactly ``pad_count`` tokens (chosen without replacement) set to -1."""
    if sequential:
        slots = np.arange(num_tokens, dtype=np.int64)
    else:
        slots = rng.choice(num_slots, size=num_tokens, replace=False).astype(np.int64)
    if pad_count:
        slots[rng.choice(num_tokens, size=pad_count, replace=False)] = -1
    return slots


@dataclass
class WriteCase:
    """Inputs of one DS-MLA cache write."""
    name: str
    kv_c: np.ndarray          # bf16 bits [T, 512]
    k_pe: np.ndarray          # bf16 bits [T, 64]
    slot_mapping: np.ndarray  # int64 [T], -1 = padding
    num_blocks: int
    block_size: int
    fill: int = 0xA5          # sentinel byte the cache is pre-filled with

    @property
    def num_tokens(self):
        return self.slot_mapping.shape[0]


@dataclass
class GatherCase:
    """Metadata of one gather-upconvert over a paged cache."""
    name: str
    block_table: np.ndarray       # int32 [B, max_blocks], -1 = unused
    workspace_starts: np.ndarray  # int32 [B], exclusive cumsum of rows per request
    seq_starts: np.ndarray        # int32 [B]
    total_tokens: int
    num_blocks: int
    block_size: int
    lengths: np.ndarray = field(default=None)  # context length per request


@dataclass
class KvWriteCase:
    """Inputs of one per-head NVFP4 K/V cache write."""
    name: str
    key: np.ndarray           # bf16 bits [T, H, hs]
    value: np.ndarray         # bf16 bits [T, H, hs]
    slot_mapping: np.ndarray  # int64 [T]
    num_blocks: int
    block_size: int
    k_scale: float            # per-tensor fp32 scales
    v_scale: float
    fill: int = 0xA5


def prefill_gather(rng, name, batch, len_lo, len_hi, num_blocks, block_size, max_blocks):
    """Requests with context length L ~ U[len_lo, len_hi], gather start
    s ~ U[0, L//2]; each request owns ceil(L/bs) consecutive entries of a
    random permutation of the cache blocks; workspace_starts is the exclusive
    cumulative sum of (L - s)."""
    L = rng.integers(len_lo, len_hi, size=batch, endpoint=True).astype(np.int64)
    s = rng.integers(0, L // 2, endpoint=True).astype(np.int64)
    perm = rng.permutation(num_blocks).astype(np.int32)
    nblk = -(-L // block_size)
    if nblk.sum() > num_blocks or nblk.max() > max_blocks:
        raise ValueError("requests do not fit the cache")
    table = np.full((batch, max_blocks), -1, np.int32)
    pos = 0
    for b in range(batch):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    rows = L - s
    ws = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int32)
    return GatherCase(name, table, ws, s.astype(np.int32), int(rows.sum()), num_blocks,
                      block_size, L)


def per_token_gather(name, slot_mapping, num_blocks, block_size):
    """One single-row request per non-padding token, in token order: request i
    reads slot_i through block_table[i] = [slot_i // bs], seq_starts = slot_i % bs."""
    valid = slot_mapping[slot_mapping >= 0]
    n = valid.shape[0]
    return GatherCase(name, (valid // block_size).astype(np.int32).reshape(n, 1),
                      np.arange(n, dtype=np.int32), (valid % block_size).astype(np.int32), n,
                      num_blocks, block_size, np.ones(n, np.int64))


# ---------------------------------------------------------------------------
# The named workloads, each with a fixed seed (tiny round trip 1001,
# decode-batch write 1002, nvfp4 prefill pair 1003, fp8 prefill pair 1004,
# per-head pair 1005).  A pre-fill write draws NoPE from stream 0 and RoPE
# from stream 2 of its seed (row-chunked, see normal_bf16_rows); the gather
# over it uses stream 1.
# ---------------------------------------------------------------------------
def tiny_round_trip():
    """Tiny round trip: 64 N(0,1) tokens, cache 8 x 64 x 352, 10% padding (6
    of 64), slots drawn from 512; gathered back per token and as one request
    over all 8 blocks."""
    rng = _rng(1001)
    kv_c = _normal_bf16(rng, (64, NOPE))
    k_pe = _normal_bf16(rng, (64, ROPE))
    slots = padded_slots(rng, 512, 64, 6)
    w = WriteCase("tiny-write", kv_c, k_pe, slots, 8, 64)
    g_tok = per_token_gather("tiny-gather-per-token", slots, 8, 64)
    g_all = GatherCase("tiny-gather-all-blocks", np.arange(8, dtype=np.int32).reshape(1, 8),
                       np.zeros(1, np.int32), np.zeros(1, np.int32), 512, 8, 64,
                       np.array([512]))
    return w, g_tok, g_all


def decode_batch_write():
    """Decode-batch write: 4096 tokens; NoPE = N(0,1) x per-token lognormal
    magnitude, 1% of elements x50; RoPE N(0,1); cache 1024 x 64; 4096 distinct
    slots of 65536, 82 (2%) padding."""
    rng = _rng(1002)
    T = 4096
    mag = np.exp(rng.standard_normal((T, 1), dtype=np.float32))
    out = np.where(rng.random((T, NOPE), dtype=np.float32) < 0.01, np.float32(50), np.float32(1))
    kv_c = bf16_bits(rng.standard_normal((T, NOPE), dtype=np.float32) * mag * out)
    k_pe = _normal_bf16(rng, (T, ROPE))
    slots = padded_slots(rng, 65536, T, 82)
    return WriteCase("decode-batch-write", kv_c, k_pe, slots, 1024, 64)


def nvfp4_prefill_write():
    """Pre-fill of the prefill-gather cache: 524288 N(0,1) tokens into every
    slot of 8192 blocks x 64 (slot_mapping = arange, no padding)."""
    T = 8192 * 64
    return WriteCase("nvfp4-prefill-write", normal_bf16_rows(1003, 0, T, NOPE),
                     normal_bf16_rows(1003, 2, T, ROPE), np.arange(T, dtype=np.int64), 8192, 64)


def nvfp4_prefill_gather():
    """Prefill gather: 16 requests, L ~ U[1024, 32768], seq_start ~ U[0, L/2],
    block tables over a shuffle of 8192 blocks (bs 64, 512 per request)."""
    return prefill_gather(_rng(1003, 1), "nvfp4-prefill-gather", 16, 1024, 32768, 8192, 64, 512)


def fp8_prefill_write():
    """fp8_ds_mla pre-fill: 1048576 N(0,1) tokens into every slot of 16384 x 64."""
    T = 16384 * 64
    return WriteCase("fp8-prefill-write", normal_bf16_rows(1004, 0, T, NOPE),
                     normal_bf16_rows(1004, 2, T, ROPE), np.arange(T, dtype=np.int64), 16384, 64)


def fp8_prefill_gather():
    """fp8_ds_mla gather: 32 requests, L ~ U[512, 16384], seq_start ~ U[0, L/2],
    block tables over a shuffle of 16384 blocks (bs 64, 256 per request)."""
    return prefill_gather(_rng(1004, 1), "fp8-prefill-gather", 32, 512, 16384, 16384, 64, 256)


def perhead_prefill_gather():
    """Per-head gather on a prefill-shaped walk over the per-head cache's 4096
    blocks of 16: 16 requests, L ~ U[512, 6144], seq_start ~ U[0, L/2], block
    tables over a shuffle of the blocks (384 per request)."""
    return prefill_gather(_rng(1005, 3), "perhead-prefill-gather", 16, 512, 6144, 4096, 16, 384)


def perhead_write_gather():
    """Per-head NVFP4 K/V write: 8192 tokens, 8 KV heads of 128, K and V each
    N(0,1) x a per-head magnitude ~ U[0.1, 10] (drawn separately for K and V);
    cache 4096 blocks x 2 x 16 x 8 x 72; 8192 distinct slots of 65536, 82 (1%)
    padding.  Per-tensor scale = amax(|side|) / 2688 (2688 = 6 * 448, so the
    largest block scale lands at the top of the e4m3 range); gathered back one
    request per non-padding token."""
    rng = _rng(1005)
    T, H, hs = 8192, 8, 128
    k_mag = rng.uniform(0.1, 10.0, size=H).astype(np.float32)
    key = bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * k_mag[None, :, None])
    v_mag = rng.uniform(0.1, 10.0, size=H).astype(np.float32)
    value = bf16_bits(rng.standard_normal((T, H, hs), dtype=np.float32) * v_mag[None, :, None])
    slots = padded_slots(rng, 4096 * 16, T, 82)
    w = KvWriteCase("perhead-write", key, value, slots, 4096, 16,
                    global_scale(key), global_scale(value))
    g = per_token_gather("perhead-gather", slots, 4096, 16)
    return w, g


def global_scale(x_bits):
    """Per-tensor scale chosen by the harness: fp32(amax(|x|)) / fp32(2688),
    or 1.0 for an all-zero tensor."""
    amax = np.float32(np.abs(bf16_to_f32(x_bits)).max()) if x_bits.size else np.float32(0)
    return float(amax / np.float32(2688.0)) if amax > 0 else 1.0


def random_write(seed, num_tokens, num_blocks, block_size, pad_count, scale=1.0):
    """A generic N(0,1)*scale write case with random distinct slots."""
    rng = _rng(seed)
    return WriteCase(f"rand-write-{seed}", bf16_bits(rng.standard_normal((num_tokens, NOPE), dtype=np.float32) * np.float32(scale)),
                     bf16_bits(rng.standard_normal((num_tokens, ROPE), dtype=np.float32) * np.float32(scale)),
                     padded_slots(rng, num_blocks * block_size, num_tokens, pad_count),
                     num_blocks, block_size)


def sparse_index_case(seed=1006, num_tokens=4096, topk=2048, batch=64, block_size=64, max_ctx=32768):
    """Top-k index rows of a sparse-attention batch: `batch` requests with
    context lengths ~ U[1024, max_ctx] and block tables over a shuffle of the
    cache blocks; every token row belongs to a request (req_id sorted, equal
    shares) and holds topk positions ~ U[0, context) with 5 % set to -1."""
    rng = _rng(seed)
    lens = rng.integers(1024, max_ctx, size=batch, endpoint=True).astype(np.int64)
    nblk = -(-lens // block_size)
    num_blocks = int(nblk.sum())
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((batch, int(-(-max_ctx // block_size))), -1, np.int32)
    pos = 0
    for b in range(batch):
        bt[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += int(nblk[b])
    req = np.sort(rng.integers(0, batch, size=num_tokens)).astype(np.int32)
    idx = (rng.random((num_tokens, topk)) * lens[req][:, None]).astype(np.int32)
    idx[rng.random((num_tokens, topk)) < 0.05] = -1
    return req, idx, bt, block_size, num_blocks
