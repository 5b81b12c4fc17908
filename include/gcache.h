/*
 * gcache.h -- C ABI of libgcache.so: quantized paged KV-cache write and
 * gather-upconvert for AMD Instinct MI355X (gfx950).
 *
 * Operations (sources are prhub.com.cn digests of three vLLM pull requests):
 *   [PR51724] "W4A16 DSA" -- nvfp4_ds_mla cache: the write
 *             concat_and_cache_nvfp4_ds_mla and the prefill gather
 *             cp_gather_and_upconvert_nvfp4_kv_cache ("Implementation
 *             breakdown" items 2-4, "Key source excerpts").
 *   [PR48642] "Sparse MLA: enable fp8_ds_mla dense prefill" -- the fp8_ds_mla
 *             gather cp_gather_and_upconvert_fp8_kv_cache with seq_starts
 *             ("Implementation breakdown" items 2 and 4, the
 *             _compute_prefill_context excerpt).
 *   [PR37332] NVFP4 per-head K/V cache for reshape_and_cache_flash
 *             ("Motivation", "Implementation breakdown" items 1 and 4,
 *             "Key source excerpts").
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every array argument is a DEVICE pointer owned by the caller (the one
 *    exception, the per-head layout struct, is a host pointer read during the
 *    call).  The library never allocates, frees or synchronizes: each call
 *    validates its arguments on the host and enqueues kernels on `stream`
 *    (which must belong to the current device).
 *  - bf16 data is IEEE bfloat16 bits; e4m3 is the OCP E4M3FN format (no
 *    infinities, 0x7F/0xFF NaN, max 448); e2m1 is OCP MX E2M1.
 *  - Strides are in ELEMENTS of the array they describe for bf16 arrays and in
 *    BYTES for the uint8 caches.  Offsets into a cache are 64-bit.
 *  - Return value: GCACHE_OK, or a negative gcache_status when an argument is
 *    rejected (nothing is launched then), when the current device is not a
 *    gfx950 GPU (GCACHE_ERR_UNSUPPORTED) or when the launch itself fails.
 *    Faults inside a kernel surface at the caller's next synchronization.
 *  - Checked inside the kernels: slot ids outside the cache are skipped like
 *    padding, and gather rows whose walk leaves the block-table row or names
 *    a block outside the cache are written as zeros, so no metadata value
 *    makes a kernel touch memory outside its arguments.
 *  - Not checked (caller contract, as in the pages' kernels): slots are
 *    distinct, workspace_starts is non-decreasing with workspace_starts[0]
 *    == 0 (otherwise rows map to unspecified requests), inputs are finite.
 *  - Calls are asynchronous and stream-ordered; two calls that write the same
 *    cache bytes on different streams race.
 *
 * Numerics (bit-exact against the CPU reference in oracle/):
 *  - NVFP4 block of 16 values x: sf = e4m3_rn_sat(amax(|x|) / 6) in binary32,
 *    inv = 1 / dec(sf) (0 when sf decodes to 0), code = e2m1_rn_sat(x * inv).
 *    The even element of a pair is the low nibble.
 *  - e4m3 RoPE: e4m3_rn_sat(r), no scale.
 *  - NVFP4 dequant: bf16(e2m1 * e4m3) -- exact, no rounding.
 */
#ifndef GCACHE_H
#define GCACHE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GCACHE_OK = 0,
    GCACHE_ERR_NULL = -1,         /* a required pointer is NULL */
    GCACHE_ERR_SHAPE = -2,        /* a size or stride is out of range */
    GCACHE_ERR_ALIGN = -3,        /* a base or stride breaks the 16-byte vector alignment */
    GCACHE_ERR_UNSUPPORTED = -4,  /* current device is not gfx950, or a shape the kernels do not cover */
    GCACHE_ERR_DEVICE = -5,       /* a HIP runtime query failed */
    GCACHE_ERR_LAUNCH = -6        /* the kernel launch failed */
} gcache_status;

typedef enum {
    GCACHE_NVFP4_DS_MLA = 0,      /* 352-byte entry */
    GCACHE_FP8_DS_MLA = 1         /* 656-byte entry */
} gcache_format;

/* Bytes per token of a DS-MLA cache entry: 352 (nvfp4_ds_mla) or 656
 * (fp8_ds_mla) -- [PR51724] "Implementation breakdown" item 2.  Returns -1
 * for an unknown format. */
int64_t gcache_entry_bytes(gcache_format format);

/* Packed last dimension of the per-head NVFP4 cache: head_size/2 data bytes
 * plus head_size/16 e4m3 scale bytes -- [PR37332] "Key source excerpts"
 * (get_kv_cache_shape).  Returns -1 unless head_size is a positive multiple
 * of 16. */
int32_t gcache_nvfp4_full_dim(int32_t head_size);

/* Human-readable name of a gcache_status value (static storage). */
const char* gcache_status_string(int status);

/*
 * Measurement hook (not part of the pages' operations; for benchmarks and
 * profilers that need a kernel's own duration).  The next kernel that an
 * entry point of this library launches from the calling host thread binds
 * `start` to the moment that kernel begins executing and `stop` to the
 * moment it ends (hipExtLaunchKernel), so hipEventElapsedTime(start, stop)
 * is the kernel's duration without the enqueue gaps that events recorded
 * around the call include.  Both events are created and owned by the caller
 * (timing enabled, on the device of the launch); either may be NULL.  The
 * hook is thread-local and consumed by that one launch: a call that is
 * rejected or launches nothing (for instance num_tokens == 0) leaves it
 * armed for the next call, and gcache_time_next_launch(NULL, NULL) disarms
 * it.  Always returns GCACHE_OK.
 */
int gcache_time_next_launch(hipEvent_t start, hipEvent_t stop);

/*
 * nvfp4_ds_mla write -- [PR51724] "Implementation breakdown" item 3 and the
 * write-kernel excerpt in "Key source excerpts".
 *
 * For every token t with slot = slot_mapping[t] >= 0, quantizes the 512 NoPE
 * values kv_c[t, 0:512] and the 64 RoPE values k_pe[t, 0:64] into the
 * 352-byte entry at
 *     kv_cache + (slot / block_size) * block_stride + (slot % block_size) * entry_stride
 * laid out as [0,256) e2m1 NoPE (16 values -> 8 bytes at 8*j for block j),
 * [256,320) e4m3 RoPE, [320,352) the 32 e4m3 NoPE block scales (scale j at
 * byte 320 + j).  Tokens with slot < 0 are padding: nothing is read or
 * written for them; a slot id >= num_blocks * block_size is skipped the same
 * way (never written out of the cache).  Bytes outside the written entries
 * are never touched.  Two tokens with the same slot race (unspecified
 * winner).
 *
 *  kv_c         bf16 [num_tokens, >=512], row stride kv_c_stride elements
 *  k_pe         bf16 [num_tokens, >=64],  row stride k_pe_stride elements
 *  kv_cache     uint8, num_blocks blocks of block_stride bytes
 *  slot_mapping int64 [num_tokens]
 * Requirements: num_tokens >= 0 (0 is a no-op), block_size > 0,
 * entry_stride >= 352, block_stride >= block_size * entry_stride;
 * kv_c and k_pe 16-byte aligned with strides that are multiples of 8
 * elements; kv_cache, block_stride and entry_stride multiples of 16 bytes.
 */
int gcache_cache_write_nvfp4_ds_mla(const void* kv_c, const void* k_pe, void* kv_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t kv_c_stride, int64_t k_pe_stride,
                                    int64_t num_blocks, int32_t block_size,
                                    int64_t block_stride, int64_t entry_stride,
                                    hipStream_t stream);

/*
 * fp8_ds_mla write -- the 656-byte entry of [PR51724] "Implementation
 * breakdown" item 2 (the pages fix only its size; the layout here is this
 * library's reading): [0,512) e4m3 NoPE codes, [512,528) four little-endian
 * fp32 scales, one per 128 values, scale = amax / 448 and code =
 * e4m3_rn_sat(x * (1 / scale)) (0 when scale is 0), [528,656) the 64 RoPE
 * values copied as bf16.  Same arguments and requirements as the nvfp4
 * write with entry_stride >= 656 (a multiple of 16).
 * Contract: a 128-value group whose amax is below 448 * 2^-126 (its
 * reciprocal scale overflows) gives unspecified codes.
 */
int gcache_cache_write_fp8_ds_mla(const void* kv_c, const void* k_pe, void* kv_cache,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  int64_t kv_c_stride, int64_t k_pe_stride,
                                  int64_t num_blocks, int32_t block_size,
                                  int64_t block_stride, int64_t entry_stride,
                                  hipStream_t stream);

/*
 * nvfp4_ds_mla gather-upconvert -- [PR51724] prefill gather excerpt
 * ("Key source excerpts"), with the seq_starts walk of [PR48642]
 * ("Implementation breakdown" item 2).
 *
 * Workspace row r (0 <= r < total_tokens) belongs to request b = the largest
 * b < batch_size with workspace_starts[b] <= r (request b owns rows
 * [ws[b], ws[b+1]); the last request ends at total_tokens, so trailing and
 * empty requests are allowed).  It reads logical position
 *     p = seq_starts[b] + (r - workspace_starts[b])      (seq_starts NULL: 0)
 * of the request, i.e. the entry at offset p % block_size of cache block
 * block_table[b * block_table_stride + p / block_size] (workspace_starts must
 * be non-decreasing with workspace_starts[0] = 0; for other values each row
 * maps to some request in [0, batch_size).  A row with p < 0,
 * p / block_size >= block_table_stride or a block id outside [0, num_blocks)
 * reads nothing and is written as zeros), and writes
 *     dst[r, 0:512]   = bf16(e2m1 * e4m3 block scale)   (exact)
 *     dst[r, 512:576] = bf16(e4m3 RoPE)                  (exact)
 *
 *  src_cache        uint8 cache written by gcache_cache_write_nvfp4_ds_mla
 *  dst              bf16 [total_tokens, >=576], row stride dst_stride elements
 *  block_table      int32 [batch_size, block_table_stride]
 *  workspace_starts int32 [batch_size]; seq_starts int32 [batch_size] or NULL
 * Requirements: total_tokens >= 0 (0 is a no-op), batch_size > 0 when
 * total_tokens > 0, dst 16-byte aligned and dst_stride a multiple of 8,
 * src_cache, block_stride and entry_stride multiples of 16 bytes,
 * entry_stride >= 352.
 */
int gcache_cache_gather_upconvert_nvfp4_ds_mla(const void* src_cache, void* dst,
                                               int64_t total_tokens, int64_t dst_stride,
                                               const int32_t* block_table,
                                               int64_t block_table_stride,
                                               const int32_t* workspace_starts,
                                               const int32_t* seq_starts, int32_t batch_size,
                                               int64_t num_blocks, int32_t block_size,
                                               int64_t block_stride, int64_t entry_stride,
                                               hipStream_t stream);

/*
 * fp8_ds_mla gather-upconvert -- [PR48642] "Implementation breakdown" items
 * 2 and 4: cp_gather_and_upconvert_fp8_kv_cache with seq_starts (seq_lens
 * removed), BF16 workspace.  Same walk and arguments as the nvfp4 gather;
 *     dst[r, i]       = bf16_rne(binary32(e4m3(code i) * scale[i / 128]))
 *     dst[r, 512:576] = the stored bf16 RoPE values
 * Requirements as for the nvfp4 gather with entry_stride >= 656.
 */
int gcache_cache_gather_upconvert_fp8_ds_mla(const void* src_cache, void* dst,
                                             int64_t total_tokens, int64_t dst_stride,
                                             const int32_t* block_table,
                                             int64_t block_table_stride,
                                             const int32_t* workspace_starts,
                                             const int32_t* seq_starts, int32_t batch_size,
                                             int64_t num_blocks, int32_t block_size,
                                             int64_t block_stride, int64_t entry_stride,
                                             hipStream_t stream);

/*
 * BF16 comparator gather -- the unquantized MLA cache that the two formats
 * above replace ([PR48642] "Key source excerpts": _compute_prefill_context
 * keeps the original bf16 gather for caches that are not fp8_ds_mla).  Same
 * walk, arguments and zero rows as the DS-MLA gathers; each entry is the
 * row's 576 bf16 values (1152 bytes, NoPE then RoPE) and is copied to
 *     dst[r, 0:576] unchanged.
 * It bounds what a walk-driven gather can reach on the device: the
 * quantized gathers read 352 or 656 bytes per row where this one reads
 * 1152.  Requirements as for the nvfp4 gather with entry_stride >= 1152.
 */
int gcache_cache_gather_bf16(const void* src_cache, void* dst, int64_t total_tokens,
                             int64_t dst_stride, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* workspace_starts,
                             const int32_t* seq_starts, int32_t batch_size, int64_t num_blocks,
                             int32_t block_size, int64_t block_stride, int64_t entry_stride,
                             hipStream_t stream);

/*
 * Sparse index conversion (triton_convert_req_index_to_global_index) --
 * [PR48642] "Implementation breakdown" item 1: a call whose req_id and
 * token_indices lengths differ is rejected (GCACHE_ERR_SHAPE) instead of
 * running past the shorter one.  For token row t and k < topk, with
 * i = token_indices[t, k] (a position in request req_id[t]'s context):
 *     out[t, k] = block_table[req_id[t], i / block_size] * block_size
 *                 + i % block_size                      (a global slot id)
 * and -1 when i < 0, req_id[t] is outside [0, batch_size), i / block_size
 * >= block_table_stride, or the block id is outside [0, num_blocks).
 *
 *  req_id         int32 [num_req_id]   (device)
 *  token_indices  int32 [num_tokens, >=topk], row stride in elements
 *  block_table    int32 [batch_size, block_table_stride]
 *  out            int32 [num_tokens, >=topk], row stride in elements
 * Requirements: num_req_id == num_tokens, num_blocks * block_size <=
 * INT32_MAX, 4-byte aligned arrays (rows 16-byte aligned with topk % 4 == 0
 * take the vector path).  num_tokens == 0 or topk == 0 is a no-op.
 */
int gcache_convert_req_index_to_global_index(const int32_t* req_id, int64_t num_req_id,
                                             const int32_t* token_indices, int64_t num_tokens,
                                             int32_t topk, int64_t token_indices_stride,
                                             const int32_t* block_table, int32_t batch_size,
                                             int64_t block_table_stride, int32_t block_size,
                                             int64_t num_blocks, int32_t* out, int64_t out_stride,
                                             hipStream_t stream);

/*
 * Chunked-context plan -- [PR48642] "Key source excerpts"
 * (_compute_prefill_context): a prefill whose cached context does not fit
 * the bf16 workspace gathers it in chunks; chunk i runs the gather with
 * workspace_starts = cu_seq_lens[i], seq_starts = starts[i] into the first
 * seq_tot[i] workspace rows.  HOST functions: every pointer is host memory,
 * nothing touches the device.
 *
 * gcache_context_chunk_plan: chunk_rows = the largest multiple of block_size
 * with batch_size * chunk_rows <= workspace_rows; num_chunks =
 * ceil(max context length / chunk_rows) (0 when every context is empty).
 * gcache_context_chunk: for chunk index `chunk`, request b gets
 *     seq_starts[b]       = chunk * chunk_rows
 *     len_b               = clamp(context_lens[b] - chunk * chunk_rows, 0, chunk_rows)
 *     workspace_starts[b] = len_0 + ... + len_{b-1},   *total_rows = sum of len_b
 * so every context position of every request is gathered exactly once, in
 * order, and no chunk needs more than workspace_rows rows.
 *  context_lens     int32 [batch_size], >= 0
 *  seq_starts, workspace_starts  int32 [batch_size] outputs
 * Errors: GCACHE_ERR_NULL for a null pointer; GCACHE_ERR_SHAPE when
 * batch_size <= 0, block_size <= 0, a context length is negative,
 * workspace_rows < batch_size * block_size, or chunk is outside
 * [0, num_chunks).
 */
int gcache_context_chunk_plan(const int32_t* context_lens, int32_t batch_size,
                              int64_t workspace_rows, int32_t block_size,
                              int32_t* chunk_rows, int32_t* num_chunks);
int gcache_context_chunk(const int32_t* context_lens, int32_t batch_size, int32_t chunk_rows,
                         int32_t chunk, int32_t* seq_starts, int32_t* workspace_starts,
                         int64_t* total_rows);

/*
 * Per-head NVFP4 K/V cache geometry, in BYTES from the start of the cache
 * ([PR37332] "Key source excerpts": allocation (num_blocks, 2, block_size,
 * num_heads, full_dim), split views into data and scale parts that keep the
 * NHD or HND order).  For block blk, side c (0 = K, 1 = V), token offset o
 * and head h:
 *   data  (head_size/2 bytes):  blk*block_stride + c*side_stride + data_offset
 *                               + o*data_token_stride + h*data_head_stride
 *   scale (head_size/16 bytes): blk*block_stride + c*side_stride + scale_offset
 *                               + o*scale_token_stride + h*scale_head_stride
 */
typedef struct {
    int64_t data_offset, data_token_stride, data_head_stride;
    int64_t scale_offset, scale_token_stride, scale_head_stride;
    int64_t side_stride, block_stride;
} gcache_nvfp4_kv_layout;

/* Fills *out with the split layout of [PR37332] ("Motivation": K data, K
 * scales, V data, V scales, each contiguous): every side of a block is all
 * data rows [block_size][num_heads][head_size/2] followed by all scale rows
 * [block_size][num_heads][head_size/16]; block_stride = 2 * block_size *
 * num_heads * full_dim.  Returns GCACHE_ERR_SHAPE for bad sizes.  The
 * per-head kernels accept the layout when block_size * num_heads * full_dim
 * (the side stride) is a multiple of 8; otherwise they return
 * GCACHE_ERR_ALIGN. */
int gcache_nvfp4_kv_split_layout(int32_t block_size, int32_t num_heads, int32_t head_size,
                                 gcache_nvfp4_kv_layout* out);

/* The same split layout in HND order ([PR37332] "Key source excerpts": the
 * split views keep the cache's NHD or HND order): inside each side, data
 * rows [num_heads][block_size][head_size/2] then scale rows
 * [num_heads][block_size][head_size/16]; same block_stride.  Returns
 * GCACHE_ERR_SHAPE for bad sizes. */
int gcache_nvfp4_kv_split_layout_hnd(int32_t block_size, int32_t num_heads, int32_t head_size,
                                     gcache_nvfp4_kv_layout* out);

/*
 * Per-head NVFP4 write (reshape_and_cache_nvfp4) -- [PR37332]
 * "Implementation breakdown" item 4.
 *
 * For every token t with 0 <= slot < num_blocks * block_size (other slot
 * ids are skipped, -1 being padding: their cache bytes are never written,
 * though their key/value rows may be read; block slot / block_size, offset
 * slot % block_size), side c in {K, V} with per-tensor scale gs (*k_scale or
 * *v_scale, device fp32 scalars > 0), head h and 16-value block j:
 *     sf = e4m3_rn_sat((amax / 6) / gs);  e = dec(sf) * gs;
 *     inv = 1 / e (0 when e is 0);        code = e2m1_rn_sat(x * inv)
 * The head's head_size/2 data bytes and head_size/16 scale bytes go to the
 * layout addresses above.
 *
 *  key, value  bf16 [num_tokens, num_heads, head_size] with the given token
 *              and head strides (elements; multiples of 8, bases 16-byte aligned)
 *  kv_cache    uint8 cache, 16-byte aligned; layout: host pointer (data_offset,
 *              the data strides, side_stride and block_stride multiples of 8
 *              bytes, else GCACHE_ERR_ALIGN; scale offset and strides any)
 * Requirements: head_size a positive multiple of 16 (at most 1024),
 * num_heads > 0, block_size > 0.
 */
int gcache_reshape_and_cache_nvfp4(const void* key, const void* value,
                                   int64_t key_token_stride, int64_t key_head_stride,
                                   int64_t value_token_stride, int64_t value_head_stride,
                                   void* kv_cache, const int64_t* slot_mapping,
                                   int64_t num_tokens, int32_t num_heads, int32_t head_size,
                                   int64_t num_blocks, int32_t block_size,
                                   const gcache_nvfp4_kv_layout* layout,
                                   const float* k_scale, const float* v_scale,
                                   hipStream_t stream);

/*
 * Per-head NVFP4 gather-upconvert -- the read side of the [PR37332] layout
 * (the pages dequantize it in test helpers, "Implementation breakdown"
 * item 5).  Same walk as the DS-MLA gathers; for every workspace row r and
 * side c:
 *     out[r, h, i] = bf16_rne(binary32((e2m1 * e4m3 block scale) * gs))
 * (rows whose walk leaves the block table or the cache are written as
 * zeros, as in the DS-MLA gathers)
 *  key_out, value_out  bf16 [total_tokens, num_heads, head_size] with token
 *                      and head strides (elements; multiples of 8, bases
 *                      16-byte aligned)
 * Other arguments as in gcache_reshape_and_cache_nvfp4 and the DS-MLA gather.
 */
int gcache_gather_upconvert_nvfp4_kv(const void* kv_cache, void* key_out, void* value_out,
                                     int64_t total_tokens,
                                     int64_t key_token_stride, int64_t key_head_stride,
                                     int64_t value_token_stride, int64_t value_head_stride,
                                     const int32_t* block_table, int64_t block_table_stride,
                                     const int32_t* workspace_starts, const int32_t* seq_starts,
                                     int32_t batch_size, int32_t num_heads, int32_t head_size,
                                     int64_t num_blocks, int32_t block_size,
                                     const gcache_nvfp4_kv_layout* layout,
                                     const float* k_scale, const float* v_scale,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GCACHE_H */
