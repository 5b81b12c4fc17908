"""CPU oracle for the quantized paged KV-cache write and gather-upconvert.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only code that may import this
package.  It wraps ``libgcache_oracle.so`` (plain C, see gcache_oracle.c) with
NumPy arrays and shares nothing with the HIP library.

bf16 tensors are passed as ``uint16`` arrays of raw bf16 bits.  Every function
raises ``OracleError`` when the C code returns a non-zero status.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))

ORC_STATUS = {0: "ok", -1: "bad argument", -2: "out of range", -3: "duplicate slot",
              -4: "non-finite input or reciprocal", -5: "invalid workspace_starts"}

NOPE_DIM, ROPE_DIM, ROW_DIM = 512, 64, 576


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status} ({ORC_STATUS.get(status, '?')})")
        self.status = status


class KvLayout(C.Structure):
    """Byte offsets/strides of the per-head NVFP4 cache (mirrors orc_kv_layout)."""
    _fields_ = [(n, C.c_int64) for n in (
        "data_offset", "data_token_stride", "data_head_stride",
        "scale_offset", "scale_token_stride", "scale_head_stride",
        "side_stride", "block_stride")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None
_P = C.c_void_p
_I64, _I32, _F32 = C.c_int64, C.c_int32, C.c_float


def lib(path=None):
    """The oracle library (built on first use).  With `path`, load and return
    that build of the same sources instead, uncached (the pin tests use it
    to check that planted mistakes are caught)."""
    global _lib
    if _lib is None or path is not None:
        L = C.CDLL(path or _build.ensure_built())
        sig = {
            "orc_e2m1_encode_array": [_P, _P, _I64], "orc_e4m3_encode_array": [_P, _P, _I64],
            "orc_f32_to_bf16_array": [_P, _P, _I64], "orc_e4m3_decode_array": [_P, _P, _I64],
            "orc_e2m1_decode_array": [_P, _P, _I64],
            "orc_write_nvfp4_ds_mla": [_P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32, _I64, _I64],
            "orc_write_fp8_ds_mla": [_P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32, _I64, _I64],
            "orc_gather_nvfp4_ds_mla": [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64, _I32,
                                        _I64, _I64],
            "orc_gather_fp8_ds_mla": [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64, _I32,
                                      _I64, _I64],
            "orc_gather_bf16": [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64, _I32,
                                _I64, _I64],
            "orc_gather_walk": [_I64, _P, _I64, _P, _P, _I32, _I64, _I32, _P, _P],
            "orc_context_chunk_plan": [_P, _I32, _I64, _I32, _P, _P],
            "orc_convert_req_index": [_P, _I64, _P, _I64, _I32, _I64, _P, _I32, _I64, _I32, _I64, _P, _I64],
            "orc_context_chunk": [_P, _I32, _I32, _I32, _P, _P, _P],
            "orc_kv_layout_split": [_I32, _I32, _I32, C.POINTER(KvLayout)],
            "orc_kv_layout_split_hnd": [_I32, _I32, _I32, C.POINTER(KvLayout)],
            "orc_reshape_and_cache_nvfp4": [_P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P, _I64, _I32,
                                            _I32, _I64, _I32, C.POINTER(KvLayout), _F32, _F32],
            "orc_gather_upconvert_nvfp4_kv": [_P, _I64, _P, _P, _I64, _I64, _I64, _I64, _I64, _P,
                                              _I64, _P, _P, _I32, _I32, _I32, _I64, _I32,
                                              C.POINTER(KvLayout), _F32, _F32],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None if name.endswith("_array") or name.startswith("orc_kv_layout_split") else C.c_int
        for name in ("orc_nvfp4_ds_mla_entry_bytes", "orc_fp8_ds_mla_entry_bytes"):
            getattr(L, name).restype = C.c_int64
            getattr(L, name).argtypes = []
        L.orc_nvfp4_full_dim.restype = C.c_int32
        L.orc_nvfp4_full_dim.argtypes = [C.c_int32]
        if path is not None:
            return L
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _need(a, dtype, name):
    if a is None:
        return None
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name}: must be C-contiguous")
    return a


def _check(status, what):
    if status != 0:
        raise OracleError(status, what)


# ---- scalar codecs, vectorised -------------------------------------------
def e2m1_encode(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e4m3_encode(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def f32_to_bf16(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(y), _ptr(out), y.size)
    return out


def e4m3_decode(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().orc_e4m3_decode_array(_ptr(codes), _ptr(out), codes.size)
    return out


def e2m1_decode(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().orc_e2m1_decode_array(_ptr(codes), _ptr(out), codes.size)
    return out


def nvfp4_ds_mla_entry_bytes():
    return lib().orc_nvfp4_ds_mla_entry_bytes()


def fp8_ds_mla_entry_bytes():
    return lib().orc_fp8_ds_mla_entry_bytes()


def nvfp4_full_dim(head_size):
    return lib().orc_nvfp4_full_dim(head_size)


# ---- DS-MLA write / gather -----------------------------------------------
def _rows(a, dtype, name):
    """2-D array whose rows may be strided (a slice of a wider buffer):
    returns the row stride in elements."""
    if a.dtype != dtype or a.ndim != 2 or a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        raise ValueError(f"{name}: expected a 2-D {np.dtype(dtype)} array with unit inner stride")
    return a.strides[0] // a.itemsize


def _write(fn, what, kv_c, k_pe, cache, slot_mapping, num_blocks, block_size,
           block_stride, entry_stride):
    kv_stride = _rows(kv_c, np.uint16, "kv_c")
    pe_stride = _rows(k_pe, np.uint16, "k_pe")
    cache = _need(cache, np.uint8, "cache")
    slot_mapping = _need(slot_mapping, np.int64, "slot_mapping")
    T = slot_mapping.shape[0]
    if kv_c.shape[0] < T or k_pe.shape[0] < T or kv_c.shape[1] < NOPE_DIM or k_pe.shape[1] < ROPE_DIM:
        raise ValueError("kv_c must be [T, >=512] and k_pe [T, >=64]")
    _check(fn(_ptr(kv_c), _ptr(k_pe), _ptr(cache), cache.size, _ptr(slot_mapping), T,
              kv_stride, pe_stride, num_blocks, block_size, block_stride, entry_stride),
           what)


def write_nvfp4_ds_mla(kv_c, k_pe, cache, slot_mapping, num_blocks, block_size,
                       block_stride=None, entry_stride=352):
    """O1: quantize kv_c [T,512] / k_pe [T,64] (bf16 bits) into cache (in place)."""
    if block_stride is None:
        block_stride = block_size * entry_stride
    _write(lib().orc_write_nvfp4_ds_mla, "write_nvfp4_ds_mla", kv_c, k_pe, cache,
           slot_mapping, num_blocks, block_size, block_stride, entry_stride)


def write_fp8_ds_mla(kv_c, k_pe, cache, slot_mapping, num_blocks, block_size,
                     block_stride=None, entry_stride=656):
    """O3: fp8_ds_mla write of kv_c [T,512] / k_pe [T,64] into cache (in place)."""
    if block_stride is None:
        block_stride = block_size * entry_stride
    _write(lib().orc_write_fp8_ds_mla, "write_fp8_ds_mla", kv_c, k_pe, cache, slot_mapping,
           num_blocks, block_size, block_stride, entry_stride)


def _gather(fn, what, cache, total_tokens, block_table, workspace_starts, seq_starts,
            num_blocks, block_size, block_stride, entry_stride, dst=None):
    cache = _need(cache, np.uint8, "cache")
    block_table = _need(block_table, np.int32, "block_table")
    workspace_starts = _need(workspace_starts, np.int32, "workspace_starts")
    seq_starts = _need(seq_starts, np.int32, "seq_starts")
    if dst is None:
        dst = np.zeros((total_tokens, ROW_DIM), np.uint16)
    _need(dst, np.uint16, "dst")
    B = workspace_starts.shape[0]
    _check(fn(_ptr(cache), cache.size, _ptr(dst), total_tokens, dst.shape[1], _ptr(block_table),
              block_table.shape[1], _ptr(workspace_starts), _ptr(seq_starts), B, num_blocks,
              block_size, block_stride, entry_stride), what)
    return dst


def gather_nvfp4_ds_mla(cache, total_tokens, block_table, workspace_starts, seq_starts,
                        num_blocks, block_size, block_stride=None, entry_stride=352, dst=None):
    """O2: gather-upconvert into a bf16-bits workspace [total_tokens, 576]."""
    if block_stride is None:
        block_stride = block_size * entry_stride
    return _gather(lib().orc_gather_nvfp4_ds_mla, "gather_nvfp4_ds_mla", cache, total_tokens,
                   block_table, workspace_starts, seq_starts, num_blocks, block_size,
                   block_stride, entry_stride, dst)


def gather_fp8_ds_mla(cache, total_tokens, block_table, workspace_starts, seq_starts,
                      num_blocks, block_size, block_stride=None, entry_stride=656, dst=None):
    """O4: fp8_ds_mla gather-upconvert into a bf16-bits workspace [total_tokens, 576]."""
    if block_stride is None:
        block_stride = block_size * entry_stride
    return _gather(lib().orc_gather_fp8_ds_mla, "gather_fp8_ds_mla", cache, total_tokens,
                   block_table, workspace_starts, seq_starts, num_blocks, block_size,
                   block_stride, entry_stride, dst)


def gather_bf16(cache, total_tokens, block_table, workspace_starts, seq_starts,
                num_blocks, block_size, block_stride=None, entry_stride=1152, dst=None):
    """BF16 comparator: the same walk over 1152-byte bf16 entries, copied."""
    if block_stride is None:
        block_stride = block_size * entry_stride
    return _gather(lib().orc_gather_bf16, "gather_bf16", cache, total_tokens,
                   block_table, workspace_starts, seq_starts, num_blocks, block_size,
                   block_stride, entry_stride, dst)


def gather_walk(total_tokens, block_table, workspace_starts, seq_starts, num_blocks, block_size):
    """(block id, offset) read by each workspace row."""
    block_table = _need(block_table, np.int32, "block_table")
    workspace_starts = _need(workspace_starts, np.int32, "workspace_starts")
    seq_starts = _need(seq_starts, np.int32, "seq_starts")
    blk = np.empty(total_tokens, np.int64)
    off = np.empty(total_tokens, np.int64)
    _check(lib().orc_gather_walk(total_tokens, _ptr(block_table), block_table.shape[1],
                                 _ptr(workspace_starts), _ptr(seq_starts),
                                 workspace_starts.shape[0], num_blocks, block_size,
                                 _ptr(blk), _ptr(off)), "gather_walk")
    return blk, off


# ---- per-head NVFP4 K/V ----------------------------------------------------
def kv_layout_split(block_size, num_heads, head_size, hnd=False):
    L = KvLayout()
    fn = lib().orc_kv_layout_split_hnd if hnd else lib().orc_kv_layout_split
    fn(block_size, num_heads, head_size, C.byref(L))
    return L


def reshape_and_cache_nvfp4(key, value, cache, slot_mapping, num_blocks, block_size,
                            layout, k_scale, v_scale):
    """O5: key/value bf16 bits [T,H,hs] -> per-head NVFP4 cache (in place)."""
    key = _need(key, np.uint16, "key")
    value = _need(value, np.uint16, "value")
    cache = _need(cache, np.uint8, "cache")
    slot_mapping = _need(slot_mapping, np.int64, "slot_mapping")
    T, H, hs = key.shape
    _check(lib().orc_reshape_and_cache_nvfp4(
        _ptr(key), _ptr(value), H * hs, hs, value.shape[1] * value.shape[2], value.shape[2],
        _ptr(cache), cache.size, _ptr(slot_mapping), slot_mapping.shape[0], H, hs, num_blocks,
        block_size, C.byref(layout), float(k_scale), float(v_scale)), "reshape_and_cache_nvfp4")


def gather_upconvert_nvfp4_kv(cache, total_tokens, block_table, workspace_starts, seq_starts,
                              num_heads, head_size, num_blocks, block_size, layout,
                              k_scale, v_scale):
    """O6: per-head gather; returns (key, value) bf16 bits [total_tokens, H, hs]."""
    cache = _need(cache, np.uint8, "cache")
    block_table = _need(block_table, np.int32, "block_table")
    workspace_starts = _need(workspace_starts, np.int32, "workspace_starts")
    seq_starts = _need(seq_starts, np.int32, "seq_starts")
    k = np.zeros((total_tokens, num_heads, head_size), np.uint16)
    v = np.zeros_like(k)
    _check(lib().orc_gather_upconvert_nvfp4_kv(
        _ptr(cache), cache.size, _ptr(k), _ptr(v), total_tokens, num_heads * head_size,
        head_size, num_heads * head_size, head_size, _ptr(block_table), block_table.shape[1],
        _ptr(workspace_starts), _ptr(seq_starts), workspace_starts.shape[0], num_heads,
        head_size, num_blocks, block_size, C.byref(layout), float(k_scale), float(v_scale)),
        "gather_upconvert_nvfp4_kv")
    return k, v


def context_chunks(context_lens, workspace_rows, block_size):
    """Chunked-context plan: (chunk_rows, [(seq_starts, workspace_starts,
    total_rows) for each chunk]) -- every context position gathered once."""
    lens = _need(np.asarray(context_lens, np.int32), np.int32, "context_lens")
    B = lens.shape[0]
    c, n = C.c_int32(), C.c_int32()
    _check(lib().orc_context_chunk_plan(_ptr(lens), B, int(workspace_rows), int(block_size),
                                        C.byref(c), C.byref(n)), "context_chunk_plan")
    out = []
    for i in range(n.value):
        ss = np.zeros(B, np.int32)
        ws = np.zeros(B, np.int32)
        tot = C.c_int64()
        _check(lib().orc_context_chunk(_ptr(lens), B, c.value, i, _ptr(ss), _ptr(ws), C.byref(tot)),
               "context_chunk")
        out.append((ss, ws, tot.value))
    return c.value, out


def convert_req_index(req_id, token_indices, block_table, block_size, num_blocks):
    """Sparse index conversion: int32 [T, topk] global slot ids (-1 invalid)."""
    req_id = _need(np.asarray(req_id, np.int32), np.int32, "req_id")
    ti = _need(np.asarray(token_indices, np.int32), np.int32, "token_indices")
    bt = _need(np.asarray(block_table, np.int32), np.int32, "block_table")
    T, K = ti.shape
    out = np.zeros((T, K), np.int32)
    _check(lib().orc_convert_req_index(_ptr(req_id), req_id.shape[0], _ptr(ti), T, K, K, _ptr(bt),
                                       bt.shape[0], bt.shape[1], int(block_size), int(num_blocks),
                                       _ptr(out), K), "convert_req_index")
    return out
