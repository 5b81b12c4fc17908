"""ctypes binding of libgcache.so (see include/gcache.h).

Argument marshalling only: tensors are checked for dtype, device and layout,
then their data pointers, strides and the current HIP stream are passed to the
C entry point of the same name (without the ``gcache_`` prefix).  Every step
of the computation runs in the HIP kernels; there is no CPU fallback, and
importing this module fails when the library has not been built.
"""
import ctypes as C
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgcache.so")

STATUS = {0: "GCACHE_OK", -1: "GCACHE_ERR_NULL", -2: "GCACHE_ERR_SHAPE", -3: "GCACHE_ERR_ALIGN",
          -4: "GCACHE_ERR_UNSUPPORTED", -5: "GCACHE_ERR_DEVICE", -6: "GCACHE_ERR_LAUNCH"}
NVFP4_DS_MLA, FP8_DS_MLA = 0, 1


class GcacheError(RuntimeError):
    def __init__(self, status, fn):
        lib = load()
        msg = lib.gcache_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class NvFp4KvLayout(C.Structure):
    """gcache_nvfp4_kv_layout: byte offsets and strides of the per-head cache."""
    _fields_ = [(n, C.c_int64) for n in (
        "data_offset", "data_token_stride", "data_head_stride",
        "scale_offset", "scale_token_stride", "scale_head_stride",
        "side_stride", "block_stride")]


_P, _I64, _I32 = C.c_void_p, C.c_int64, C.c_int32
_SIGS = {
    "gcache_entry_bytes": (_I64, [C.c_int]),
    "gcache_nvfp4_full_dim": (_I32, [_I32]),
    "gcache_status_string": (C.c_char_p, [C.c_int]),
    "gcache_time_next_launch": (C.c_int, [_P, _P]),
    "gcache_cache_write_nvfp4_ds_mla": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I64, _I64, _P]),
    "gcache_cache_write_fp8_ds_mla": (C.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I64, _I64, _P]),
    "gcache_cache_gather_upconvert_nvfp4_ds_mla": (C.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64,
                                                            _I32, _I64, _I64, _P]),
    "gcache_cache_gather_upconvert_fp8_ds_mla": (C.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64,
                                                          _I32, _I64, _I64, _P]),
    "gcache_cache_gather_bf16": (C.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _I32, _I64, _I32, _I64,
                                           _I64, _P]),
    "gcache_nvfp4_kv_split_layout": (C.c_int, [_I32, _I32, _I32, C.POINTER(NvFp4KvLayout)]),
    "gcache_nvfp4_kv_split_layout_hnd": (C.c_int, [_I32, _I32, _I32, C.POINTER(NvFp4KvLayout)]),
    "gcache_context_chunk_plan": (C.c_int, [_P, _I32, _I64, _I32, _P, _P]),
    "gcache_convert_req_index_to_global_index": (C.c_int, [_P, _I64, _P, _I64, _I32, _I64, _P, _I32, _I64,
                                                           _I32, _I64, _P, _I64, _P]),
    "gcache_context_chunk": (C.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "gcache_reshape_and_cache_nvfp4": (C.c_int, [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _I64, _I32, _I32, _I64,
                                                 _I32, C.POINTER(NvFp4KvLayout), _P, _P, _P]),
    "gcache_gather_upconvert_nvfp4_kv": (C.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _P, _P,
                                                   _I32, _I32, _I32, _I64, _I32, C.POINTER(NvFp4KvLayout), _P,
                                                   _P, _P]),
}

_lib = None


def load():
    """Load libgcache.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python gather_concat_cache_amd/build.py` (hipcc, gfx950)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(status, fn):
    if status != 0:
        raise GcacheError(status, fn)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(t, dtype, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def time_next_launch(start_event, stop_event):
    """Bind the next kernel that this library launches from the calling
    thread to two HIP events (raw hipEvent_t handles as integers, or None):
    `start_event` records when that kernel begins, `stop_event` when it ends
    (gcache_time_next_launch)."""
    _check(load().gcache_time_next_launch(start_event, stop_event), "time_next_launch")


def entry_bytes(fmt):
    """Bytes per token: 352 for NVFP4_DS_MLA, 656 for FP8_DS_MLA."""
    return load().gcache_entry_bytes(fmt)


def nvfp4_full_dim(head_size):
    return load().gcache_nvfp4_full_dim(head_size)


def nvfp4_kv_split_layout(block_size, num_heads, head_size, hnd=False):
    """Split per-head NVFP4 layout (data rows then scale rows in each side),
    NHD token-major, or HND head-major with hnd=True."""
    L = NvFp4KvLayout()
    name = "gcache_nvfp4_kv_split_layout_hnd" if hnd else "gcache_nvfp4_kv_split_layout"
    _check(getattr(load(), name)(block_size, num_heads, head_size, C.byref(L)), name)
    return L


def nvfp4_kv_split_views(kv_cache, num_heads, head_size, layout=None):
    """Views of a per-head NVFP4 cache (uint8, num_blocks x block_size
    given by kv_cache.shape[0] and kv_cache.shape[2] of the
    (num_blocks, 2, block_size, num_heads, full_dim) allocation):
    ([k_data, v_data], [k_scale, v_scale]) as uint8 [num_blocks, block_size,
    num_heads, head_size/2] and float8_e4m3fn [num_blocks, block_size,
    num_heads, head_size/16] over the same bytes, for any layout (default
    the NHD split layout).  Works on CPU and GPU tensors alike."""
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 5:
        raise ValueError("kv_cache must be uint8 [num_blocks, 2, block_size, num_heads, full_dim]")
    nb, bs = kv_cache.shape[0], kv_cache.shape[2]
    if layout is None:
        layout = nvfp4_kv_split_layout(bs, num_heads, head_size)
    base = kv_cache.as_strided((kv_cache.untyped_storage().nbytes() - kv_cache.storage_offset(),), (1,))
    if _layout_extent(layout, nb, bs, num_heads, head_size) > base.numel():
        raise ValueError("layout reaches past the cache allocation")
    data, scale = [], []
    for side in (0, 1):
        o = side * layout.side_stride
        data.append(base.as_strided((nb, bs, num_heads, head_size // 2),
                                    (layout.block_stride, layout.data_token_stride, layout.data_head_stride, 1),
                                    base.storage_offset() + o + layout.data_offset))
        scale.append(base.as_strided((nb, bs, num_heads, head_size // 16),
                                     (layout.block_stride, layout.scale_token_stride, layout.scale_head_stride, 1),
                                     base.storage_offset() + o + layout.scale_offset).view(torch.float8_e4m3fn))
    return data, scale


# ---------------------------------------------------------------------------
def _ds_cache_geometry(kv_cache, name):
    """kv_cache: uint8 [num_blocks, block_size, entry_stride-or-more] with unit
    last stride -> (num_blocks, block_size, block_stride, entry_stride)."""
    if kv_cache.dim() != 3 or kv_cache.stride(2) != 1:
        raise ValueError(f"{name}: expected uint8 [num_blocks, block_size, entry] with unit last stride")
    return kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0), kv_cache.stride(1)


def _ds_write(fn_name, kv_c, k_pe, kv_cache, slot_mapping, stream):
    dev = _dev_tensor(kv_cache, torch.uint8, "kv_cache").device
    _dev_tensor(kv_c, torch.bfloat16, "kv_c", dev)
    _dev_tensor(k_pe, torch.bfloat16, "k_pe", dev)
    _dev_tensor(slot_mapping, torch.int64, "slot_mapping", dev)
    T = slot_mapping.numel()
    if T == 0:
        return                                   # no tokens: nothing to do
    if kv_c.dim() != 2 or k_pe.dim() != 2 or kv_c.stride(1) != 1 or k_pe.stride(1) != 1:
        raise ValueError("kv_c and k_pe must be 2-D with unit last stride")
    if kv_c.shape[0] < T or k_pe.shape[0] < T or kv_c.shape[1] < 512 or k_pe.shape[1] < 64:
        raise ValueError("kv_c must be [T, >=512] and k_pe [T, >=64]")
    if not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous")
    nb, bs, bstr, estr = _ds_cache_geometry(kv_cache, "kv_cache")
    with torch.cuda.device(dev):
        st = getattr(load(), fn_name)(_ptr(kv_c), _ptr(k_pe), _ptr(kv_cache), _ptr(slot_mapping), T,
                                      kv_c.stride(0), k_pe.stride(0), nb, bs, bstr, estr,
                                      _stream(dev, stream))
    _check(st, fn_name)


def cache_write_nvfp4_ds_mla(kv_c, k_pe, kv_cache, slot_mapping, stream=None):
    """Quantize kv_c bf16 [T,512] and k_pe bf16 [T,64] into the nvfp4_ds_mla
    cache uint8 [num_blocks, block_size, >=352] at slot_mapping (int64 [T],
    < 0 skipped).  Enqueued on the current stream (or `stream`)."""
    _ds_write("gcache_cache_write_nvfp4_ds_mla", kv_c, k_pe, kv_cache, slot_mapping, stream)


def cache_write_fp8_ds_mla(kv_c, k_pe, kv_cache, slot_mapping, stream=None):
    """fp8_ds_mla write into uint8 [num_blocks, block_size, >=656]."""
    _ds_write("gcache_cache_write_fp8_ds_mla", kv_c, k_pe, kv_cache, slot_mapping, stream)


def _check_walk_args(block_table, workspace_starts, seq_starts, batch_size):
    """Shared checks of the gather walk's metadata; returns the batch size.
    The block table's row stride is also the bound the kernels apply to a
    row's block index, so its rows must be contiguous."""
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    if workspace_starts.dim() != 1 or not workspace_starts.is_contiguous() or \
            (seq_starts is not None and (seq_starts.dim() != 1 or not seq_starts.is_contiguous())):
        raise ValueError("workspace_starts / seq_starts must be contiguous int32 vectors")
    B = workspace_starts.numel() if batch_size is None else int(batch_size)
    if B > workspace_starts.numel() or (seq_starts is not None and B > seq_starts.numel()) \
            or B > block_table.shape[0]:
        raise ValueError("batch_size exceeds workspace_starts / seq_starts / block_table")
    return B


def _ds_gather(fn_name, src_cache, dst, block_table, workspace_starts, seq_starts, batch_size, stream):
    dev = _dev_tensor(src_cache, torch.uint8, "src_cache").device
    _dev_tensor(dst, torch.bfloat16, "dst", dev)
    _dev_tensor(block_table, torch.int32, "block_table", dev)
    _dev_tensor(workspace_starts, torch.int32, "workspace_starts", dev)
    if seq_starts is not None:
        _dev_tensor(seq_starts, torch.int32, "seq_starts", dev)
    if dst.dim() == 2 and dst.shape[0] == 0:
        return                                   # no rows: nothing to do
    if dst.dim() != 2 or dst.stride(1) != 1 or dst.shape[1] < 576:
        raise ValueError("dst must be bf16 [total_tokens, >=576] with unit last stride")
    B = _check_walk_args(block_table, workspace_starts, seq_starts, batch_size)
    nb, bs, bstr, estr = _ds_cache_geometry(src_cache, "src_cache")
    with torch.cuda.device(dev):
        st = getattr(load(), fn_name)(_ptr(src_cache), _ptr(dst), dst.shape[0], dst.stride(0),
                                      _ptr(block_table), block_table.stride(0), _ptr(workspace_starts),
                                      _ptr(seq_starts), B, nb, bs, bstr, estr, _stream(dev, stream))
    _check(st, fn_name)


def cache_gather_upconvert_nvfp4_ds_mla(src_cache, dst, block_table, workspace_starts,
                                        seq_starts=None, batch_size=None, stream=None):
    """Gather-upconvert nvfp4_ds_mla entries into dst bf16 [total_tokens, 576]:
    row r of request b (ws[b] <= r < ws[b+1]) reads position
    seq_starts[b] + r - ws[b] through block_table[b]."""
    _ds_gather("gcache_cache_gather_upconvert_nvfp4_ds_mla", src_cache, dst, block_table,
               workspace_starts, seq_starts, batch_size, stream)


def cache_gather_upconvert_fp8_ds_mla(src_cache, dst, block_table, workspace_starts,
                                      seq_starts=None, batch_size=None, stream=None):
    """fp8_ds_mla gather-upconvert into dst bf16 [total_tokens, 576]."""
    _ds_gather("gcache_cache_gather_upconvert_fp8_ds_mla", src_cache, dst, block_table,
               workspace_starts, seq_starts, batch_size, stream)


def cache_gather_bf16(src_cache, dst, block_table, workspace_starts, seq_starts=None, batch_size=None,
                      stream=None):
    """BF16 comparator: the same walk over a bf16 cache [num_blocks, block_size,
    >=576] (unit last stride), rows copied into dst bf16 [total_tokens, 576]."""
    if not isinstance(src_cache, torch.Tensor) or src_cache.dtype != torch.bfloat16 \
            or src_cache.dim() != 3 or src_cache.stride(2) != 1:
        raise ValueError("src_cache must be a bf16 [num_blocks, block_size, >=576] tensor with unit last stride")
    _ds_gather("gcache_cache_gather_bf16", src_cache.view(torch.uint8), dst, block_table, workspace_starts,
               seq_starts, batch_size, stream)


# ---------------------------------------------------------------------------
def _kv_geometry(kv_cache, num_heads, head_size, layout):
    """kv_cache uint8 [num_blocks, 2, block_size, H, full_dim] -> (nb, bs, layout)."""
    if kv_cache.dim() != 5 or kv_cache.shape[1] != 2:
        raise ValueError("kv_cache must be uint8 [num_blocks, 2, block_size, num_heads, full_dim]")
    nb, bs = kv_cache.shape[0], kv_cache.shape[2]
    if layout is None:
        if not kv_cache.is_contiguous():
            raise ValueError("the default split layout needs a contiguous kv_cache")
        layout = nvfp4_kv_split_layout(bs, num_heads, head_size)
    avail = kv_cache.untyped_storage().nbytes() - kv_cache.storage_offset()
    if _layout_extent(layout, nb, bs, num_heads, head_size) > avail:
        raise ValueError("the layout addresses bytes past the kv_cache allocation")
    return nb, bs, layout


def _layout_extent(layout, nb, bs, num_heads, head_size):
    """One past the last cache byte the layout addresses for nb blocks."""
    if nb == 0:
        return 0
    side = max(layout.data_offset + (bs - 1) * layout.data_token_stride
               + (num_heads - 1) * layout.data_head_stride + head_size // 2,
               layout.scale_offset + (bs - 1) * layout.scale_token_stride
               + (num_heads - 1) * layout.scale_head_stride + head_size // 16)
    return (nb - 1) * layout.block_stride + layout.side_stride + side


def _scale(t, name, dev):
    _dev_tensor(t, torch.float32, name, dev)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold one fp32 value")
    return t


def reshape_and_cache_nvfp4(key, value, kv_cache, slot_mapping, k_scale, v_scale, layout=None,
                            stream=None):
    """Per-head NVFP4 write of key / value bf16 [T, H, hs] into kv_cache uint8
    [num_blocks, 2, block_size, H, hs/2 + hs/16] (split layout unless a
    NvFp4KvLayout is given); k_scale / v_scale: fp32 device scalars."""
    dev = _dev_tensor(kv_cache, torch.uint8, "kv_cache").device
    _dev_tensor(key, torch.bfloat16, "key", dev)
    _dev_tensor(value, torch.bfloat16, "value", dev)
    _dev_tensor(slot_mapping, torch.int64, "slot_mapping", dev)
    _scale(k_scale, "k_scale", dev)
    _scale(v_scale, "v_scale", dev)
    if key.dim() != 3 or value.shape != key.shape or key.stride(2) != 1 or value.stride(2) != 1:
        raise ValueError("key / value must be bf16 [T, H, hs] with unit last stride")
    T, H, hs = key.shape
    if slot_mapping.numel() == 0:
        return
    if slot_mapping.numel() > T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous with at most T entries")
    nb, bs, layout = _kv_geometry(kv_cache, H, hs, layout)
    with torch.cuda.device(dev):
        st = load().gcache_reshape_and_cache_nvfp4(
            _ptr(key), _ptr(value), key.stride(0), key.stride(1), value.stride(0), value.stride(1),
            _ptr(kv_cache), _ptr(slot_mapping), slot_mapping.numel(), H, hs, nb, bs, C.byref(layout),
            _ptr(k_scale), _ptr(v_scale), _stream(dev, stream))
    _check(st, "reshape_and_cache_nvfp4")


def gather_upconvert_nvfp4_kv(kv_cache, key_out, value_out, block_table, workspace_starts,
                              k_scale, v_scale, seq_starts=None, batch_size=None, layout=None,
                              stream=None):
    """Per-head NVFP4 gather-upconvert into key_out / value_out bf16
    [total_tokens, H, hs] through the DS-MLA gather walk."""
    dev = _dev_tensor(kv_cache, torch.uint8, "kv_cache").device
    _dev_tensor(key_out, torch.bfloat16, "key_out", dev)
    _dev_tensor(value_out, torch.bfloat16, "value_out", dev)
    _dev_tensor(block_table, torch.int32, "block_table", dev)
    _dev_tensor(workspace_starts, torch.int32, "workspace_starts", dev)
    if seq_starts is not None:
        _dev_tensor(seq_starts, torch.int32, "seq_starts", dev)
    _scale(k_scale, "k_scale", dev)
    _scale(v_scale, "v_scale", dev)
    if key_out.dim() != 3 or value_out.shape != key_out.shape or key_out.stride(2) != 1 \
            or value_out.stride(2) != 1:
        raise ValueError("key_out / value_out must be bf16 [total, H, hs] with unit last stride")
    total, H, hs = key_out.shape
    if total == 0:
        return
    B = _check_walk_args(block_table, workspace_starts, seq_starts, batch_size)
    nb, bs, layout = _kv_geometry(kv_cache, H, hs, layout)
    with torch.cuda.device(dev):
        st = load().gcache_gather_upconvert_nvfp4_kv(
            _ptr(kv_cache), _ptr(key_out), _ptr(value_out), total, key_out.stride(0), key_out.stride(1),
            value_out.stride(0), value_out.stride(1), _ptr(block_table), block_table.stride(0),
            _ptr(workspace_starts), _ptr(seq_starts), B, H, hs, nb, bs, C.byref(layout),
            _ptr(k_scale), _ptr(v_scale), _stream(dev, stream))
    _check(st, "gather_upconvert_nvfp4_kv")


# ---------------------------------------------------------------------------
# chunked context (host plan from the library, gathers on the device)
# ---------------------------------------------------------------------------
def context_chunks(context_lens, workspace_rows, block_size):
    """Host plan of a chunked-context gather: (chunk_rows, [(seq_starts,
    workspace_starts, total_rows), ...]) as int32 NumPy arrays."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    B = lens.shape[0]
    lib = load()
    c, n = C.c_int32(), C.c_int32()
    _check(lib.gcache_context_chunk_plan(lens.ctypes.data, B, int(workspace_rows), int(block_size),
                                         C.addressof(c), C.addressof(n)), "gcache_context_chunk_plan")
    chunks = []
    for i in range(n.value):
        ss = np.empty(B, np.int32)
        ws = np.empty(B, np.int32)
        tot = C.c_int64()
        _check(lib.gcache_context_chunk(lens.ctypes.data, B, c.value, i, ss.ctypes.data, ws.ctypes.data,
                                        C.addressof(tot)), "gcache_context_chunk")
        chunks.append((ss, ws, tot.value))
    return c.value, chunks


def gather_context_chunked(gather, src_cache, workspace, block_table, context_lens, stream=None):
    """Gather every request's whole cached context (positions 0 ..
    context_lens[b]-1) through a bounded bf16 workspace [rows, >=576], one
    chunk at a time.  `gather` is one of cache_gather_upconvert_nvfp4_ds_mla,
    cache_gather_upconvert_fp8_ds_mla or cache_gather_bf16.  Yields
    (chunk index, workspace[:total_rows]) after enqueuing each chunk's gather
    on the stream; consume (or copy) a chunk before asking for the next one,
    which overwrites the workspace.  All chunks' metadata is uploaded once."""
    lens = np.asarray(context_lens, dtype=np.int32)
    block_size = src_cache.shape[1]
    _, chunks = context_chunks(lens, workspace.shape[0], block_size)
    if not chunks:
        return
    # one upload of every chunk's metadata [chunks, 2, B] from pinned host
    # memory, ordered on the stream before the first gather
    host_meta = torch.from_numpy(np.stack([np.stack([ss, ws]) for ss, ws, _ in chunks])).pin_memory()
    s = torch.cuda.current_stream(workspace.device) if stream is None else stream
    with torch.cuda.stream(s):
        meta = host_meta.to(workspace.device, non_blocking=True)
    for i, (_, _, total) in enumerate(chunks):
        rows = workspace[:total]
        gather(src_cache, rows, block_table, meta[i, 1], meta[i, 0], stream=stream)
        yield i, rows


# ---------------------------------------------------------------------------
# sparse index conversion
# ---------------------------------------------------------------------------
def convert_req_index_to_global_index(req_id, token_indices, block_table, block_size, num_blocks,
                                      out=None, stream=None):
    """Top-k positions local to each token's request -> global slot ids:
    out[t, k] = block_table[req_id[t], i // block_size] * block_size + i % block_size
    for i = token_indices[t, k], -1 where invalid.  req_id int32 [T] must have
    exactly one entry per token row (the call is rejected otherwise);
    token_indices int32 [T, topk]; block_table int32 [batch, max_blocks].
    Returns out (int32 [T, topk], allocated when not given)."""
    dev = _dev_tensor(token_indices, torch.int32, "token_indices").device
    _dev_tensor(req_id, torch.int32, "req_id", dev)
    _dev_tensor(block_table, torch.int32, "block_table", dev)
    if token_indices.dim() != 2 or token_indices.stride(1) != 1:
        raise ValueError("token_indices must be int32 [num_tokens, topk] with unit last stride")
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [batch, max_blocks] tensor")
    if req_id.dim() != 1 or req_id.stride(0) != 1:
        raise ValueError("req_id must be a contiguous int32 vector")
    T, K = token_indices.shape
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=dev)
    _dev_tensor(out, torch.int32, "out", dev)
    if out.dim() != 2 or out.shape[0] != T or out.shape[1] < K or out.stride(1) != 1:
        raise ValueError("out must be int32 [num_tokens, >=topk] with unit last stride")
    with torch.cuda.device(dev):
        st = load().gcache_convert_req_index_to_global_index(
            _ptr(req_id), req_id.shape[0], _ptr(token_indices), T, K, token_indices.stride(0),
            _ptr(block_table), block_table.shape[0], block_table.stride(0), int(block_size), int(num_blocks),
            _ptr(out), out.stride(0), _stream(dev, stream))
    _check(st, "gcache_convert_req_index_to_global_index")
    return out
