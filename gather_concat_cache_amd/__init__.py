"""gather_concat_cache_amd -- quantized paged KV-cache write and gather-upconvert
for AMD Instinct MI355X (gfx950).

The computation lives in libgcache.so (hand-written HIP kernels behind the C
ABI of include/gcache.h); this package only marshals torch tensors (device
memory and streams) into those calls.  Each function is exported under the
C name and under the C name without the ``gcache_`` prefix.
"""
from ._native import (FP8_DS_MLA, LIB_PATH, NVFP4_DS_MLA, GcacheError, NvFp4KvLayout,
                      cache_gather_bf16, cache_gather_upconvert_fp8_ds_mla, cache_gather_upconvert_nvfp4_ds_mla,
                      cache_write_fp8_ds_mla, cache_write_nvfp4_ds_mla, context_chunks,
                      convert_req_index_to_global_index, entry_bytes,
                      gather_context_chunked,
                      gather_upconvert_nvfp4_kv, load, nvfp4_full_dim, nvfp4_kv_split_layout, nvfp4_kv_split_views,
                      reshape_and_cache_nvfp4, time_next_launch)

__all__ = [
    "NVFP4_DS_MLA", "FP8_DS_MLA", "LIB_PATH", "GcacheError", "NvFp4KvLayout", "load",
    "entry_bytes", "nvfp4_full_dim", "nvfp4_kv_split_layout", "nvfp4_kv_split_views",
    "cache_write_nvfp4_ds_mla", "cache_write_fp8_ds_mla",
    "cache_gather_upconvert_nvfp4_ds_mla", "cache_gather_upconvert_fp8_ds_mla", "cache_gather_bf16",
    "reshape_and_cache_nvfp4", "gather_upconvert_nvfp4_kv",
    "context_chunks", "gather_context_chunked", "convert_req_index_to_global_index", "time_next_launch",
]

# The same functions under the C entry points' own names.
gcache_entry_bytes = entry_bytes
gcache_nvfp4_full_dim = nvfp4_full_dim
gcache_nvfp4_kv_split_layout = nvfp4_kv_split_layout
gcache_cache_write_nvfp4_ds_mla = cache_write_nvfp4_ds_mla
gcache_cache_write_fp8_ds_mla = cache_write_fp8_ds_mla
gcache_cache_gather_upconvert_nvfp4_ds_mla = cache_gather_upconvert_nvfp4_ds_mla
gcache_cache_gather_upconvert_fp8_ds_mla = cache_gather_upconvert_fp8_ds_mla
gcache_cache_gather_bf16 = cache_gather_bf16
gcache_reshape_and_cache_nvfp4 = reshape_and_cache_nvfp4
gcache_gather_upconvert_nvfp4_kv = gather_upconvert_nvfp4_kv
gcache_convert_req_index_to_global_index = convert_req_index_to_global_index
gcache_time_next_launch = time_next_launch
__all__ += [n for n in list(globals()) if n.startswith("gcache_")]

load()   # fail at import time when libgcache.so has not been built
