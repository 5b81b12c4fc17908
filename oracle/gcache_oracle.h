/*
 * gcache_oracle.h -- CPU reference ("oracle") for the quantized DS-MLA and
 * per-head NVFP4 paged KV-cache write and gather-upconvert.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only code allowed to load this.
 * It shares no code, header, table or constant with the HIP library
 * (include/gcache.h, gather_concat_cache_amd/csrc); neither side includes
 * the other.  Everything here is plain, scalar and slow on purpose: each
 * step follows the rule it implements so that a reader can check it by eye.
 *
 * Sources (cited by page and section; the pages are prhub.com.cn digests of
 * three vLLM pull requests):
 *   [P1] vLLM PR #51724 digest -- "W4A16 DSA": nvfp4_ds_mla cache format,
 *        write kernel concat_and_cache_nvfp4_ds_mla and prefill gather
 *        cp_gather_and_upconvert_nvfp4_kv_cache.
 *   [P2] vLLM PR #37332 digest -- NVFP4 per-head KV cache for
 *        reshape_and_cache_flash; full_dim / split-view helpers.
 *   [P3] vLLM PR #48642 digest -- fp8_ds_mla dense prefill fix; the gather
 *        gains seq_starts.
 * Element formats follow the OCP Microscaling (MX) v1.0 definitions of
 * E2M1 and E4M3 (the "fn" variant: no infinities, S.1111.111 is NaN) and
 * IEEE-754 binary32 round-to-nearest-even.
 *
 * Readings taken where the pages are silent are marked READING in the .c
 * file.
 *
 * Parity status: every function below is pinned by the CPU test suite
 * (exhaustive codec sweeps against an independent bit-level encoder,
 * nearest-value brute force, torch's float8_e4m3fn / bfloat16 casts,
 * hand-derived vectors, the pages' own tolerances, and NumPy brute-force
 * round trips).  The scale-byte order inside the 352-byte entry (identity)
 * and the per-head scale swizzle (identity) are readings with no third-party
 * reader to compare against: parity unpinned for those two choices only.
 */
#ifndef GCACHE_ORACLE_H
#define GCACHE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ORC_OK             0
#define ORC_ERR_ARG       -1  /* null pointer, negative size, bad stride */
#define ORC_ERR_RANGE     -2  /* slot, block id or address outside the cache */
#define ORC_ERR_DUP       -3  /* two tokens map to the same slot */
#define ORC_ERR_NONFINITE -4  /* input outside the finite contract */
#define ORC_ERR_WALK      -5  /* workspace_starts not a valid partition */

/* ---- scalar codecs -------------------------------------------------- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16_rne(float f);
uint8_t  orc_e2m1_encode(float y);     /* RN-even, satfinite, sign kept  */
float    orc_e2m1_decode(uint8_t code);
uint8_t  orc_e4m3_encode(float y);     /* OCP E4M3FN, RN-even, satfinite */
float    orc_e4m3_decode(uint8_t code);

/* array forms, for the test harness (n elements each) */
void orc_e2m1_encode_array(const float* in, uint8_t* out, int64_t n);
void orc_e4m3_encode_array(const float* in, uint8_t* out, int64_t n);
void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n);
void orc_e4m3_decode_array(const uint8_t* in, float* out, int64_t n);
void orc_e2m1_decode_array(const uint8_t* in, float* out, int64_t n);

/* ---- entry geometry ------------------------------------------------- */
int64_t orc_nvfp4_ds_mla_entry_bytes(void);      /* 352 */
int64_t orc_fp8_ds_mla_entry_bytes(void);        /* 656 */
int32_t orc_nvfp4_full_dim(int32_t head_size);   /* hs/2 + hs/16 */

/* ---- O1: nvfp4_ds_mla write ----------------------------------------- */
/* kv_c: bf16 bits [num_tokens, >=512] with row stride kv_c_stride elements;
 * k_pe: bf16 bits [num_tokens, >=64] with row stride k_pe_stride elements;
 * cache: cache_bytes bytes, entry of slot s at
 *        (s / block_size) * block_stride + (s % block_size) * entry_stride. */
int orc_write_nvfp4_ds_mla(const uint16_t* kv_c, const uint16_t* k_pe,
                           uint8_t* cache, int64_t cache_bytes,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           int64_t kv_c_stride, int64_t k_pe_stride,
                           int64_t num_blocks, int32_t block_size,
                           int64_t block_stride, int64_t entry_stride);

/* ---- O3: fp8_ds_mla write (same arguments, 656-byte entries) -------- */
int orc_write_fp8_ds_mla(const uint16_t* kv_c, const uint16_t* k_pe,
                         uint8_t* cache, int64_t cache_bytes,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int64_t kv_c_stride, int64_t k_pe_stride,
                         int64_t num_blocks, int32_t block_size,
                         int64_t block_stride, int64_t entry_stride);

/* ---- O2 / O4: gather-upconvert into a bf16 workspace ---------------- */
/* dst: bf16 bits [total_tokens, >=576], row stride dst_stride elements.
 * Request b owns workspace rows [ws[b], ws[b+1]) (the last one ends at
 * total_tokens); row r of request b reads logical position
 * seq_starts[b] + (r - ws[b]) of that request (seq_starts may be NULL = 0). */
int orc_gather_nvfp4_ds_mla(const uint8_t* cache, int64_t cache_bytes,
                            uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* workspace_starts, const int32_t* seq_starts,
                            int32_t batch_size, int64_t num_blocks, int32_t block_size,
                            int64_t block_stride, int64_t entry_stride);
int orc_gather_fp8_ds_mla(const uint8_t* cache, int64_t cache_bytes,
                          uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                          const int32_t* block_table, int64_t block_table_stride,
                          const int32_t* workspace_starts, const int32_t* seq_starts,
                          int32_t batch_size, int64_t num_blocks, int32_t block_size,
                          int64_t block_stride, int64_t entry_stride);

/* BF16 comparator: the same walk over a cache of 1152-byte entries holding
 * the row's 576 bf16 values; rows are copied unchanged. */
int orc_gather_bf16(const uint8_t* cache, int64_t cache_bytes,
                    uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* workspace_starts, const int32_t* seq_starts,
                    int32_t batch_size, int64_t num_blocks, int32_t block_size,
                    int64_t block_stride, int64_t entry_stride);

/* Walk only: for each workspace row, the (block id, offset in block) that
 * the gather reads.  out_block / out_offset have total_tokens entries. */
int orc_gather_walk(int64_t total_tokens,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* workspace_starts, const int32_t* seq_starts,
                    int32_t batch_size, int64_t num_blocks, int32_t block_size,
                    int64_t* out_block, int64_t* out_offset);

/* ---- O5 / O6: per-head NVFP4 K/V ------------------------------------ */
/* Byte address of head h, token offset o, side c (0 = K, 1 = V) in block blk:
 *   data : blk*block_stride + c*side_stride + data_offset
 *          + o*data_token_stride + h*data_head_stride      (head_size/2 bytes)
 *   scale: blk*block_stride + c*side_stride + scale_offset
 *          + o*scale_token_stride + h*scale_head_stride    (head_size/16 bytes) */
typedef struct {
    int64_t data_offset, data_token_stride, data_head_stride;
    int64_t scale_offset, scale_token_stride, scale_head_stride;
    int64_t side_stride, block_stride;
} orc_kv_layout;

/* The split layout of the per-head cache (K side then V side; each side is
 * all data rows followed by all scale rows, token-major). */
void orc_kv_layout_split(int32_t block_size, int32_t num_heads, int32_t head_size,
                         orc_kv_layout* out);
void orc_kv_layout_split_hnd(int32_t block_size, int32_t num_heads, int32_t head_size,
                             orc_kv_layout* out);

/* key/value: bf16 bits [num_tokens, num_heads, head_size] with the given
 * token and head strides (elements); k_scale / v_scale: per-tensor fp32. */
int orc_reshape_and_cache_nvfp4(const uint16_t* key, const uint16_t* value,
                                int64_t key_token_stride, int64_t key_head_stride,
                                int64_t value_token_stride, int64_t value_head_stride,
                                uint8_t* cache, int64_t cache_bytes,
                                const int64_t* slot_mapping, int64_t num_tokens,
                                int32_t num_heads, int32_t head_size,
                                int64_t num_blocks, int32_t block_size,
                                const orc_kv_layout* layout,
                                float k_scale, float v_scale);

int orc_gather_upconvert_nvfp4_kv(const uint8_t* cache, int64_t cache_bytes,
                                  uint16_t* key_out, uint16_t* value_out,
                                  int64_t total_tokens,
                                  int64_t key_token_stride, int64_t key_head_stride,
                                  int64_t value_token_stride, int64_t value_head_stride,
                                  const int32_t* block_table, int64_t block_table_stride,
                                  const int32_t* workspace_starts, const int32_t* seq_starts,
                                  int32_t batch_size, int32_t num_heads, int32_t head_size,
                                  int64_t num_blocks, int32_t block_size,
                                  const orc_kv_layout* layout,
                                  float k_scale, float v_scale);

/* ---- chunked context plan (host metadata of a chunked prefill) ------ */
/* chunk_rows: largest multiple of block_size with batch_size * chunk_rows
 * <= workspace_rows; position p of a request is gathered by chunk
 * p / chunk_rows, whose rows hold requests one after another. */
int orc_context_chunk_plan(const int32_t* context_lens, int32_t batch_size,
                           int64_t workspace_rows, int32_t block_size,
                           int32_t* chunk_rows, int32_t* num_chunks);
int orc_context_chunk(const int32_t* context_lens, int32_t batch_size, int32_t chunk_rows,
                      int32_t chunk, int32_t* seq_starts, int32_t* workspace_starts,
                      int64_t* total_rows);

/* ---- sparse index conversion ---------------------------------------- */
/* out[t, k] = global slot of position token_indices[t, k] of request
 * req_id[t] (block_table[req][i / bs] * bs + i % bs), -1 when invalid;
 * ORC_ERR_ARG when num_req_id != num_tokens. */
int orc_convert_req_index(const int32_t* req_id, int64_t num_req_id,
                          const int32_t* token_indices, int64_t num_tokens, int32_t topk,
                          int64_t token_indices_stride, const int32_t* block_table,
                          int32_t batch_size, int64_t block_table_stride, int32_t block_size,
                          int64_t num_blocks, int32_t* out, int64_t out_stride);

#ifdef __cplusplus
}
#endif
#endif /* GCACHE_ORACLE_H */
