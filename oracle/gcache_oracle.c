/*
 * gcache_oracle.c -- CPU reference for the quantized paged KV-cache write and
 * gather-upconvert.  TEST INFRASTRUCTURE ONLY (see gcache_oracle.h): only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * Plain scalar C.  Floating-point steps that the method performs in binary32
 * are written as binary32 C expressions (one IEEE rounding each; build with
 * -ffp-contract=off and without fast-math so nothing is fused or reordered).
 * Steps that are exact (decoding, the NVFP4 dequant product) are exact here.
 */
#include "gcache_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Entry geometry.                                                            */
/* vLLM PR #51724 digest, "Implementation breakdown" item 3: one 352-byte     */
/* nvfp4_ds_mla entry holds 256 B of packed e2m1 NoPE, then 64 B of e4m3      */
/* RoPE, then 32 B of e4m3 NoPE scales, in that order.  Item 2 of the same    */
/* section gives the per-token sizes 656 (fp8_ds_mla) and 352 (nvfp4_ds_mla). */
/* The NoPE width 512 and RoPE width 64 are the DS-MLA shapes the write test  */
/* in "Key source excerpts" requires (kv_lora_rank must be 512).              */
/* ------------------------------------------------------------------------ */
enum {
    NOPE_DIM = 512,
    ROPE_DIM = 64,
    ROW_DIM = NOPE_DIM + ROPE_DIM,        /* gathered workspace row: 576 */

    NV_BLOCK = 16,                        /* NVFP4: one scale per 16 values */
    NV_NOPE_BYTES = NOPE_DIM / 2,         /* 256: two e2m1 codes per byte   */
    NV_ROPE_OFF = NV_NOPE_BYTES,          /* 256 */
    NV_ROPE_BYTES = ROPE_DIM,             /* 64 e4m3 codes, no scale        */
    NV_SCALE_OFF = NV_ROPE_OFF + NV_ROPE_BYTES,   /* 320 */
    NV_SCALE_BYTES = NOPE_DIM / NV_BLOCK,         /* 32 */
    NV_ENTRY = NV_SCALE_OFF + NV_SCALE_BYTES,     /* 352 */

    /* READING (fp8_ds_mla internals; the pages give only the 656 total):
     * 512 e4m3 NoPE codes, four little-endian fp32 scales (one per 128
     * values, scale = amax / 448), then the 64 RoPE values as raw bf16. */
    F8_GROUP = 128,
    F8_SCALE_OFF = NOPE_DIM,                       /* 512 */
    F8_SCALE_BYTES = 4 * (NOPE_DIM / F8_GROUP),    /* 16  */
    F8_ROPE_OFF = F8_SCALE_OFF + F8_SCALE_BYTES,   /* 528 */
    F8_ENTRY = F8_ROPE_OFF + 2 * ROPE_DIM          /* 656 */
};

int64_t orc_nvfp4_ds_mla_entry_bytes(void) { return NV_ENTRY; }
int64_t orc_fp8_ds_mla_entry_bytes(void) { return F8_ENTRY; }

/* vLLM PR #37332 digest, "Key source excerpts" (flashinfer.py,
 * get_kv_cache_shape): the packed last dimension of the per-head NVFP4
 * cache is head_size/2 bytes of fp4 data plus head_size/16 scale bytes. */
int32_t orc_nvfp4_full_dim(int32_t head_size) { return head_size / 2 + head_size / 16; }

/* READING: the digest of PR #51724 says the kernel permutes the NoPE scale
 * factors but does not print the permutation.  Identity is used: scale j
 * covers NoPE elements 16j .. 16j+15 and is stored at byte 320 + j. */
static int nope_scale_position(int j) { return j; }

/* ------------------------------------------------------------------------ */
/* Scalar codecs.                                                             */
/* ------------------------------------------------------------------------ */
static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the upper half of a binary32: widening is exact. */
float orc_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/* Round a binary32 to bf16, nearest, ties to even.  Two same-sign floats
 * whose bit patterns differ by one are adjacent values, so the 16 dropped
 * bits measure linearly how far f sits between the truncated bf16 t and the
 * next one away from zero, t + 1 (also across a binade edge). */
uint16_t orc_f32_to_bf16_rne(float f) {
    uint32_t u = f32_to_bits(f);
    if (isnan(f)) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t t = u >> 16;
    uint32_t rem = u & 0xFFFFu;
    if (rem > 0x8000u) return (uint16_t)(t + 1);
    if (rem < 0x8000u) return (uint16_t)t;
    return (uint16_t)((t & 1u) ? t + 1 : t);       /* exact tie: even */
}

/* E2M1 (OCP MX): sign, 2 exponent bits with bias 1, 1 mantissa bit.
 * Exponent field 0 is subnormal: value = m * 0.5. */
float orc_e2m1_decode(uint8_t code) {
    int e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m / 2.0, e - 1);
    return (float)((code & 8) ? -mag : mag);
}

/* E4M3FN (OCP): sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities; magnitude code 0x7F is NaN.  Exponent field 0 is subnormal:
 * value = m * 2^-9.  Largest finite magnitude 0x7E = 1.75 * 2^8 = 448. */
float orc_e4m3_decode(uint8_t code) {
    int e = (code >> 3) & 15, m = code & 7;
    if ((code & 0x7F) == 0x7F) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)((code & 0x80) ? -mag : mag);
}

/* Non-negative magnitude tables in code order (magnitudes increase with the
 * code in both formats).  Filled from the decoders above when the library
 * is loaded, before any caller (or caller thread) can use them. */
static double e2m1_mag[8];
static double e4m3_mag[127];

__attribute__((constructor)) static void build_tables(void) {
    for (int c = 0; c < 8; c++) e2m1_mag[c] = orc_e2m1_decode((uint8_t)c);
    for (int c = 0; c < 127; c++) e4m3_mag[c] = orc_e4m3_decode((uint8_t)c);
}

/* Round-to-nearest with ties to the even code (mantissa LSB 0), saturating
 * at the largest finite magnitude.  a >= 0.  The midpoint of two adjacent
 * grid values has at most 5 significant bits, so it is exact in double and
 * the comparison with the float a decides the rounding exactly. */
static int nearest_code(double a, const double* mag, int ncodes) {
    if (a >= mag[ncodes - 1]) return ncodes - 1;             /* satfinite */
    int lo = 0, hi = ncodes - 1;                             /* mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mag[mid] <= a) lo = mid; else hi = mid;
    }
    double midpoint = (mag[lo] + mag[hi]) / 2.0;
    if (a < midpoint) return lo;
    if (a > midpoint) return hi;
    return (lo % 2 == 0) ? lo : hi;                          /* tie -> even */
}

/* e2m1 RN-even satfinite; the sign bit is the sign of y, so -0 and small
 * negatives encode as 0x8.  NaN has no e2m1 code: 0xFF flags it. */
uint8_t orc_e2m1_encode(float y) {
    if (isnan(y)) return 0xFF;
    int mag = nearest_code(fabs((double)y), e2m1_mag, 8);
    return (uint8_t)((signbit(y) ? 8 : 0) | mag);
}

/* e4m3fn RN-even satfinite (|y| >= 448 -> 448, infinities included); the
 * sign is kept, so values that round to zero give 0x00 / 0x80. */
uint8_t orc_e4m3_encode(float y) {
    if (isnan(y)) return (uint8_t)((signbit(y) ? 0x80 : 0) | 0x7F);
    int mag = nearest_code(fabs((double)y), e4m3_mag, 127);
    return (uint8_t)((signbit(y) ? 0x80 : 0) | mag);
}

void orc_e2m1_encode_array(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_e2m1_encode(in[i]);
}
void orc_e4m3_encode_array(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_encode(in[i]);
}
void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16_rne(in[i]);
}
void orc_e4m3_decode_array(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_decode(in[i]);
}
void orc_e2m1_decode_array(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_e2m1_decode(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Shared validation helpers.                                                 */
/* ------------------------------------------------------------------------ */
static int bf16_is_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

/* Slot decoding: vLLM PR #51724 digest, "Key source excerpts" (the write
 * kernel): a negative slot marks a padding token that is skipped; otherwise
 * block = slot / block_size and offset = slot % block_size, and the entry
 * sits at block * block_stride + offset * entry_stride. */
static int64_t slot_address(int64_t slot, int32_t block_size,
                            int64_t block_stride, int64_t entry_stride) {
    return (slot / block_size) * block_stride + (slot % block_size) * entry_stride;
}

/* Range and duplicate check of a slot mapping (READING: duplicate slots make
 * the writes race; the oracle refuses them). */
static int check_slots(const int64_t* slot_mapping, int64_t num_tokens,
                       int64_t num_blocks, int32_t block_size) {
    int64_t nslots = num_blocks * (int64_t)block_size;
    unsigned char* seen = (unsigned char*)calloc((size_t)(nslots / 8 + 1), 1);
    if (!seen) return ORC_ERR_ARG;
    int rc = ORC_OK;
    for (int64_t t = 0; t < num_tokens && rc == ORC_OK; t++) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        if (s >= nslots) { rc = ORC_ERR_RANGE; break; }
        if (seen[s / 8] & (1u << (s % 8))) { rc = ORC_ERR_DUP; break; }
        seen[s / 8] |= (unsigned char)(1u << (s % 8));
    }
    free(seen);
    return rc;
}

static int check_ds_mla_geometry(int64_t num_tokens, int64_t kv_c_stride, int64_t k_pe_stride,
                                 int64_t num_blocks, int32_t block_size,
                                 int64_t block_stride, int64_t entry_stride,
                                 int64_t entry_bytes, int64_t cache_bytes) {
    if (num_tokens < 0 || num_blocks < 0 || block_size <= 0) return ORC_ERR_ARG;
    if (kv_c_stride < NOPE_DIM || k_pe_stride < ROPE_DIM) return ORC_ERR_ARG;
    if (entry_stride < entry_bytes) return ORC_ERR_ARG;
    if (block_stride < (int64_t)block_size * entry_stride) return ORC_ERR_ARG;
    if (num_blocks > 0 && (num_blocks - 1) * block_stride
                          + (int64_t)(block_size - 1) * entry_stride + entry_bytes > cache_bytes)
        return ORC_ERR_RANGE;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* O1: nvfp4_ds_mla write.                                                    */
/* vLLM PR #51724 digest, "Key source excerpts" (nvfp4_ds_mla_cache_kernels): */
/* NoPE is handled 16 consecutive values at a time: a block scale from the   */
/* block's absolute maximum, then the values times the reciprocal scale are  */
/* rounded to e2m1 (RN, satfinite) and packed 16 values to 8 bytes at byte   */
/* 8 * block; RoPE is cast to e4m3 without a scale.  The test in the same    */
/* section compares the scale bytes with a reference built from amax and the */
/* e2m1 maximum 6.0, and dequantizes as code * scale repeated per 16 values. */
/* ------------------------------------------------------------------------ */
static void quantize_nvfp4_token(const uint16_t* nope, const uint16_t* rope, uint8_t* entry) {
    uint8_t q[NOPE_DIM];
    for (int j = 0; j < NOPE_DIM / NV_BLOCK; j++) {
        float x[NV_BLOCK];
        float amax = 0.0f;
        for (int i = 0; i < NV_BLOCK; i++) {
            x[i] = orc_bf16_to_f32(nope[j * NV_BLOCK + i]);
            if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
        }
        /* READING: scale = e4m3_rn_sat(amax / 6) in binary32; the values are
         * multiplied by the binary32 reciprocal of the decoded scale (0 when
         * the scale is 0) and then rounded to e2m1. */
        uint8_t sf = orc_e4m3_encode(amax / 6.0f);
        float s = orc_e4m3_decode(sf);
        float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
        for (int i = 0; i < NV_BLOCK; i++) q[j * NV_BLOCK + i] = orc_e2m1_encode(x[i] * inv);
        entry[NV_SCALE_OFF + nope_scale_position(j)] = sf;
    }
    /* READING: the even element sits in the low nibble of each byte. */
    for (int k = 0; k < NV_NOPE_BYTES; k++)
        entry[k] = (uint8_t)(q[2 * k] | (q[2 * k + 1] << 4));
    for (int i = 0; i < ROPE_DIM; i++)
        entry[NV_ROPE_OFF + i] = orc_e4m3_encode(orc_bf16_to_f32(rope[i]));
}

int orc_write_nvfp4_ds_mla(const uint16_t* kv_c, const uint16_t* k_pe,
                           uint8_t* cache, int64_t cache_bytes,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           int64_t kv_c_stride, int64_t k_pe_stride,
                           int64_t num_blocks, int32_t block_size,
                           int64_t block_stride, int64_t entry_stride) {
    int rc = check_ds_mla_geometry(num_tokens, kv_c_stride, k_pe_stride, num_blocks, block_size,
                                   block_stride, entry_stride, NV_ENTRY, cache_bytes);
    if (rc) return rc;
    if (num_tokens == 0) return ORC_OK;
    if (!kv_c || !k_pe || !cache || !slot_mapping) return ORC_ERR_ARG;
    if ((rc = check_slots(slot_mapping, num_tokens, num_blocks, block_size))) return rc;
    for (int64_t t = 0; t < num_tokens; t++) {          /* finite inputs only */
        if (slot_mapping[t] < 0) continue;
        for (int i = 0; i < NOPE_DIM; i++)
            if (!bf16_is_finite(kv_c[t * kv_c_stride + i])) return ORC_ERR_NONFINITE;
        for (int i = 0; i < ROPE_DIM; i++)
            if (!bf16_is_finite(k_pe[t * k_pe_stride + i])) return ORC_ERR_NONFINITE;
    }
    for (int64_t t = 0; t < num_tokens; t++) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;                          /* padding token */
        uint8_t entry[NV_ENTRY];
        quantize_nvfp4_token(kv_c + t * kv_c_stride, k_pe + t * k_pe_stride, entry);
        memcpy(cache + slot_address(slot, block_size, block_stride, entry_stride), entry, NV_ENTRY);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* O3: fp8_ds_mla write (656-byte entry; internals are a READING, see the    */
/* geometry enum above).  Per 128-value group: scale = amax / 448 stored as  */
/* binary32, codes = e4m3_rn_sat(x * (1 / scale)) (0 when scale is 0).       */
/* ------------------------------------------------------------------------ */
static int fp8_group_scale(const uint16_t* nope, int g, float* scale, float* inv) {
    float amax = 0.0f;
    for (int i = 0; i < F8_GROUP; i++) {
        float x = orc_bf16_to_f32(nope[g * F8_GROUP + i]);
        if (fabsf(x) > amax) amax = fabsf(x);
    }
    *scale = amax / 448.0f;
    *inv = (*scale == 0.0f) ? 0.0f : 1.0f / *scale;
    return isfinite(*inv) ? ORC_OK : ORC_ERR_NONFINITE;   /* amax below the contract */
}

int orc_write_fp8_ds_mla(const uint16_t* kv_c, const uint16_t* k_pe,
                         uint8_t* cache, int64_t cache_bytes,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int64_t kv_c_stride, int64_t k_pe_stride,
                         int64_t num_blocks, int32_t block_size,
                         int64_t block_stride, int64_t entry_stride) {
    int rc = check_ds_mla_geometry(num_tokens, kv_c_stride, k_pe_stride, num_blocks, block_size,
                                   block_stride, entry_stride, F8_ENTRY, cache_bytes);
    if (rc) return rc;
    if (num_tokens == 0) return ORC_OK;
    if (!kv_c || !k_pe || !cache || !slot_mapping) return ORC_ERR_ARG;
    if ((rc = check_slots(slot_mapping, num_tokens, num_blocks, block_size))) return rc;
    for (int64_t t = 0; t < num_tokens; t++) {
        if (slot_mapping[t] < 0) continue;
        const uint16_t* nope = kv_c + t * kv_c_stride;
        for (int i = 0; i < NOPE_DIM; i++)
            if (!bf16_is_finite(nope[i])) return ORC_ERR_NONFINITE;
        for (int i = 0; i < ROPE_DIM; i++)
            if (!bf16_is_finite(k_pe[t * k_pe_stride + i])) return ORC_ERR_NONFINITE;
        for (int g = 0; g < NOPE_DIM / F8_GROUP; g++) {
            float sc, inv;
            if ((rc = fp8_group_scale(nope, g, &sc, &inv))) return rc;
        }
    }
    for (int64_t t = 0; t < num_tokens; t++) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const uint16_t* nope = kv_c + t * kv_c_stride;
        const uint16_t* rope = k_pe + t * k_pe_stride;
        uint8_t entry[F8_ENTRY];
        for (int g = 0; g < NOPE_DIM / F8_GROUP; g++) {
            float sc, inv;
            fp8_group_scale(nope, g, &sc, &inv);
            for (int i = g * F8_GROUP; i < (g + 1) * F8_GROUP; i++)
                entry[i] = orc_e4m3_encode(orc_bf16_to_f32(nope[i]) * inv);
            uint32_t bits = f32_to_bits(sc);
            for (int k = 0; k < 4; k++)                        /* little endian */
                entry[F8_SCALE_OFF + 4 * g + k] = (uint8_t)(bits >> (8 * k));
        }
        for (int i = 0; i < ROPE_DIM; i++) {                   /* bf16 copied as is */
            entry[F8_ROPE_OFF + 2 * i] = (uint8_t)(rope[i] & 0xFF);
            entry[F8_ROPE_OFF + 2 * i + 1] = (uint8_t)(rope[i] >> 8);
        }
        memcpy(cache + slot_address(slot, block_size, block_stride, entry_stride), entry, F8_ENTRY);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Gather walk.                                                               */
/* vLLM PR #51724 digest, "Key source excerpts" (the prefill gather): each   */
/* output row finds its request among workspace_starts, then the cache       */
/* address through that request's block table.  vLLM PR #48642 digest,      */
/* "Implementation breakdown" item 2 and the _compute_prefill_context        */
/* excerpt: seq_starts lets a request's gather begin at any cache position.  */
/* READING: request b owns rows [ws[b], ws[b+1]) and the last one ends at     */
/* total_tokens; row r of request b reads logical position                   */
/* seq_starts[b] + (r - ws[b]) of the request's block table.                 */
/* ------------------------------------------------------------------------ */
static int check_walk_args(int64_t total_tokens, const int32_t* block_table,
                           int64_t block_table_stride, const int32_t* workspace_starts,
                           int32_t batch_size, int32_t block_size) {
    if (total_tokens < 0 || block_size <= 0) return ORC_ERR_ARG;
    if (total_tokens == 0) return ORC_OK;
    if (!block_table || !workspace_starts || batch_size <= 0 || block_table_stride <= 0)
        return ORC_ERR_ARG;
    if (workspace_starts[0] != 0) return ORC_ERR_WALK;      /* every row has a request */
    for (int32_t b = 1; b < batch_size; b++)
        if (workspace_starts[b] < workspace_starts[b - 1]) return ORC_ERR_WALK;
    return ORC_OK;
}

/* One row: the request is the largest b with ws[b] <= r (a plain scan). */
static int walk_row(int64_t r, const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* ws, const int32_t* seq_starts, int32_t batch_size,
                    int64_t num_blocks, int32_t block_size, int64_t* blk, int64_t* off) {
    int32_t req = -1;
    for (int32_t b = 0; b < batch_size; b++)
        if (ws[b] <= r) req = b;
    if (req < 0) return ORC_ERR_WALK;
    int64_t pos = (int64_t)(seq_starts ? seq_starts[req] : 0) + (r - ws[req]);
    if (pos < 0 || pos / block_size >= block_table_stride) return ORC_ERR_RANGE;
    int64_t id = block_table[(int64_t)req * block_table_stride + pos / block_size];
    if (id < 0 || id >= num_blocks) return ORC_ERR_RANGE;
    *blk = id;
    *off = pos % block_size;
    return ORC_OK;
}

int orc_gather_walk(int64_t total_tokens,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* workspace_starts, const int32_t* seq_starts,
                    int32_t batch_size, int64_t num_blocks, int32_t block_size,
                    int64_t* out_block, int64_t* out_offset) {
    int rc = check_walk_args(total_tokens, block_table, block_table_stride, workspace_starts,
                             batch_size, block_size);
    if (rc) return rc;
    for (int64_t r = 0; r < total_tokens; r++) {
        rc = walk_row(r, block_table, block_table_stride, workspace_starts, seq_starts,
                      batch_size, num_blocks, block_size, &out_block[r], &out_offset[r]);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Shared driver of the two DS-MLA gathers: validate every row first, then
 * decode entry by entry. */
typedef void (*row_decoder)(const uint8_t* entry, uint16_t* row);

static int gather_ds_mla(const uint8_t* cache, int64_t cache_bytes, uint16_t* dst,
                         int64_t total_tokens, int64_t dst_stride,
                         const int32_t* block_table, int64_t block_table_stride,
                         const int32_t* ws, const int32_t* seq_starts, int32_t batch_size,
                         int64_t num_blocks, int32_t block_size, int64_t block_stride,
                         int64_t entry_stride, int64_t entry_bytes, row_decoder decode) {
    if (total_tokens < 0 || block_size <= 0 || num_blocks < 0) return ORC_ERR_ARG;
    if (entry_stride < entry_bytes || block_stride < (int64_t)block_size * entry_stride)
        return ORC_ERR_ARG;
    if (total_tokens == 0) return ORC_OK;
    if (!cache || !dst || dst_stride < ROW_DIM) return ORC_ERR_ARG;
    int rc = check_walk_args(total_tokens, block_table, block_table_stride, ws, batch_size,
                             block_size);
    if (rc) return rc;
    for (int64_t r = 0; r < total_tokens; r++) {
        int64_t blk, off;
        rc = walk_row(r, block_table, block_table_stride, ws, seq_starts, batch_size,
                      num_blocks, block_size, &blk, &off);
        if (rc) return rc;
        if (blk * block_stride + off * entry_stride + entry_bytes > cache_bytes)
            return ORC_ERR_RANGE;
    }
    for (int64_t r = 0; r < total_tokens; r++) {
        int64_t blk, off;
        walk_row(r, block_table, block_table_stride, ws, seq_starts, batch_size, num_blocks,
                 block_size, &blk, &off);
        decode(cache + blk * block_stride + off * entry_stride, dst + r * dst_stride);
    }
    return ORC_OK;
}

/* O2 row: NoPE value i = e2m1(nibble i) * e4m3(scale of block i/16); the
 * product has at most 6 significant bits and lies in [2^-10, 2688], so it is
 * exact in binary32 and in bf16 (the bf16 rounding below never rounds).
 * RoPE value i = e4m3 code i widened to bf16 (also exact).  Columns: NoPE
 * 0..511 then RoPE 512..575 (the write takes NoPE first, RoPE second). */
static void decode_nvfp4_row(const uint8_t* entry, uint16_t* row) {
    for (int i = 0; i < NOPE_DIM; i++) {
        uint8_t byte = entry[i / 2];
        uint8_t nib = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        uint8_t sf = entry[NV_SCALE_OFF + nope_scale_position(i / NV_BLOCK)];
        double v = (double)orc_e2m1_decode(nib) * (double)orc_e4m3_decode(sf);
        row[i] = orc_f32_to_bf16_rne((float)v);
    }
    for (int i = 0; i < ROPE_DIM; i++)
        row[NOPE_DIM + i] = orc_f32_to_bf16_rne(orc_e4m3_decode(entry[NV_ROPE_OFF + i]));
}

/* O4 row: NoPE value i = bf16_rne(binary32(e4m3(code i) * scale of group
 * i/128)) -- READING: one binary32 multiply, then one rounding to bf16.
 * RoPE bf16 values are copied. */
static void decode_fp8_row(const uint8_t* entry, uint16_t* row) {
    float sc[NOPE_DIM / F8_GROUP];
    for (int g = 0; g < NOPE_DIM / F8_GROUP; g++) {
        uint32_t bits = 0;
        for (int k = 0; k < 4; k++) bits |= (uint32_t)entry[F8_SCALE_OFF + 4 * g + k] << (8 * k);
        sc[g] = bits_to_f32(bits);
    }
    for (int i = 0; i < NOPE_DIM; i++) {
        float v = orc_e4m3_decode(entry[i]) * sc[i / F8_GROUP];
        row[i] = orc_f32_to_bf16_rne(v);
    }
    for (int i = 0; i < ROPE_DIM; i++)
        row[NOPE_DIM + i] = (uint16_t)(entry[F8_ROPE_OFF + 2 * i]
                                       | (entry[F8_ROPE_OFF + 2 * i + 1] << 8));
}

int orc_gather_nvfp4_ds_mla(const uint8_t* cache, int64_t cache_bytes,
                            uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* workspace_starts, const int32_t* seq_starts,
                            int32_t batch_size, int64_t num_blocks, int32_t block_size,
                            int64_t block_stride, int64_t entry_stride) {
    return gather_ds_mla(cache, cache_bytes, dst, total_tokens, dst_stride, block_table,
                         block_table_stride, workspace_starts, seq_starts, batch_size,
                         num_blocks, block_size, block_stride, entry_stride, NV_ENTRY,
                         decode_nvfp4_row);
}

int orc_gather_fp8_ds_mla(const uint8_t* cache, int64_t cache_bytes,
                          uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                          const int32_t* block_table, int64_t block_table_stride,
                          const int32_t* workspace_starts, const int32_t* seq_starts,
                          int32_t batch_size, int64_t num_blocks, int32_t block_size,
                          int64_t block_stride, int64_t entry_stride) {
    return gather_ds_mla(cache, cache_bytes, dst, total_tokens, dst_stride, block_table,
                         block_table_stride, workspace_starts, seq_starts, batch_size,
                         num_blocks, block_size, block_stride, entry_stride, F8_ENTRY,
                         decode_fp8_row);
}

/* BF16 comparator (the plain bf16 MLA cache that the quantized formats
 * replace; vLLM PR #48642 digest, the _compute_prefill_context excerpt,
 * keeps it as the path for unquantized caches): the same walk, each
 * 1152-byte entry holds the row's 576 bf16 values (NoPE then RoPE, little
 * endian) and is copied unchanged. */
static void copy_bf16_row(const uint8_t* entry, uint16_t* row) {
    for (int i = 0; i < ROW_DIM; i++)
        row[i] = (uint16_t)(entry[2 * i] | (entry[2 * i + 1] << 8));
}

int orc_gather_bf16(const uint8_t* cache, int64_t cache_bytes,
                    uint16_t* dst, int64_t total_tokens, int64_t dst_stride,
                    const int32_t* block_table, int64_t block_table_stride,
                    const int32_t* workspace_starts, const int32_t* seq_starts,
                    int32_t batch_size, int64_t num_blocks, int32_t block_size,
                    int64_t block_stride, int64_t entry_stride) {
    return gather_ds_mla(cache, cache_bytes, dst, total_tokens, dst_stride, block_table,
                         block_table_stride, workspace_starts, seq_starts, batch_size,
                         num_blocks, block_size, block_stride, entry_stride, 2 * ROW_DIM,
                         copy_bf16_row);
}


/* ------------------------------------------------------------------------ */
/* O5 / O6: per-head NVFP4 K/V cache.                                        */
/* vLLM PR #37332 digest: "Motivation" and "Implementation breakdown" item 4 */
/* describe a K/V cache whose pages hold K data, K scales, V data, V scales  */
/* (fp4 data, one e4m3 scale per 16 values, plus a per-tensor scale);        */
/* "Key source excerpts" give the allocation (num_blocks, 2, block_size,     */
/* num_heads, full_dim) and split views that separate data and scale bytes   */
/* (data = full_dim * 8 / 9) while keeping the NHD or HND order.             */
/* READING (split layout): each side of a block is all data rows             */
/* [block_size][num_heads][head_size/2] followed by all scale rows           */
/* [block_size][num_heads][head_size/16]; any other arrangement is expressed */
/* through the offsets and strides of orc_kv_layout.                          */
/* READING (global scale gs, a dequant multiplier): block scale              */
/* sf = e4m3_rn_sat((amax / 6) / gs); effective scale e = dec(sf) * gs;      */
/* codes = e2m1_rn_sat(x * (1 / e)) (0 when e is 0); dequant value =        */
/* bf16_rne(binary32((e2m1 * e4m3) * gs)).  READING: no scale swizzle.       */
/* ------------------------------------------------------------------------ */
void orc_kv_layout_split(int32_t block_size, int32_t num_heads, int32_t head_size,
                         orc_kv_layout* out) {
    int64_t data_row = head_size / 2, scale_row = head_size / 16;
    int64_t side = (int64_t)block_size * num_heads * (data_row + scale_row);
    out->data_offset = 0;
    out->data_token_stride = (int64_t)num_heads * data_row;
    out->data_head_stride = data_row;
    out->scale_offset = (int64_t)block_size * num_heads * data_row;
    out->scale_token_stride = (int64_t)num_heads * scale_row;
    out->scale_head_stride = scale_row;
    out->side_stride = side;
    out->block_stride = 2 * side;
}

/* HND order of the split layout: within a side, head h's data rows for all
 * token offsets come before head h+1's, then the scale rows in the same
 * order (vLLM PR #37332 digest, "Key source excerpts": the split views keep
 * NHD or HND).  Written as sizes of the nested regions. */
void orc_kv_layout_split_hnd(int32_t block_size, int32_t num_heads, int32_t head_size,
                             orc_kv_layout* out) {
    int64_t data_row = head_size / 2, scale_row = head_size / 16;
    int64_t data_per_head = block_size * data_row;          /* one head, all offsets */
    int64_t scale_per_head = block_size * scale_row;
    int64_t data_region = num_heads * data_per_head;
    int64_t scale_region = num_heads * scale_per_head;
    out->data_offset = 0;
    out->data_head_stride = data_per_head;
    out->data_token_stride = data_row;
    out->scale_offset = data_region;
    out->scale_head_stride = scale_per_head;
    out->scale_token_stride = scale_row;
    out->side_stride = data_region + scale_region;
    out->block_stride = 2 * out->side_stride;
}

static int check_kv_args(int64_t num_tokens, int32_t num_heads, int32_t head_size,
                         int64_t num_blocks, int32_t block_size, const orc_kv_layout* L,
                         int64_t cache_bytes, float k_scale, float v_scale) {
    if (!L || num_tokens < 0 || num_heads <= 0 || head_size <= 0 || head_size % 16 != 0 ||
        num_blocks < 0 || block_size <= 0)
        return ORC_ERR_ARG;
    if (!(isfinite(k_scale) && k_scale > 0.0f && isfinite(v_scale) && v_scale > 0.0f))
        return ORC_ERR_ARG;
    if (L->data_offset < 0 || L->scale_offset < 0 || L->data_token_stride < 0 ||
        L->data_head_stride < 0 || L->scale_token_stride < 0 || L->scale_head_stride < 0 ||
        L->side_stride < 0 || L->block_stride < 0)
        return ORC_ERR_ARG;
    if (num_blocks == 0) return ORC_OK;
    int64_t last = (num_blocks - 1) * L->block_stride + L->side_stride;
    int64_t data_end = last + L->data_offset + (int64_t)(block_size - 1) * L->data_token_stride
                       + (int64_t)(num_heads - 1) * L->data_head_stride + head_size / 2;
    int64_t scale_end = last + L->scale_offset + (int64_t)(block_size - 1) * L->scale_token_stride
                        + (int64_t)(num_heads - 1) * L->scale_head_stride + head_size / 16;
    if (data_end > cache_bytes || scale_end > cache_bytes) return ORC_ERR_RANGE;
    return ORC_OK;
}

/* Quantize one head row of head_size values into its data and scale bytes. */
static int quantize_kv_head(const uint16_t* x, int32_t head_size, float gs,
                            uint8_t* data, uint8_t* scales) {
    for (int j = 0; j < head_size / NV_BLOCK; j++) {
        float v[NV_BLOCK];
        float amax = 0.0f;
        for (int i = 0; i < NV_BLOCK; i++) {
            v[i] = orc_bf16_to_f32(x[j * NV_BLOCK + i]);
            if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
        }
        uint8_t sf = orc_e4m3_encode((amax / 6.0f) / gs);
        float e = orc_e4m3_decode(sf) * gs;
        float inv = (e == 0.0f) ? 0.0f : 1.0f / e;
        if (!isfinite(inv)) return ORC_ERR_NONFINITE;
        uint8_t q[NV_BLOCK];
        for (int i = 0; i < NV_BLOCK; i++) q[i] = orc_e2m1_encode(v[i] * inv);
        for (int k = 0; k < NV_BLOCK / 2; k++)
            data[j * (NV_BLOCK / 2) + k] = (uint8_t)(q[2 * k] | (q[2 * k + 1] << 4));
        scales[j] = sf;
    }
    return ORC_OK;
}

int orc_reshape_and_cache_nvfp4(const uint16_t* key, const uint16_t* value,
                                int64_t key_token_stride, int64_t key_head_stride,
                                int64_t value_token_stride, int64_t value_head_stride,
                                uint8_t* cache, int64_t cache_bytes,
                                const int64_t* slot_mapping, int64_t num_tokens,
                                int32_t num_heads, int32_t head_size,
                                int64_t num_blocks, int32_t block_size,
                                const orc_kv_layout* L, float k_scale, float v_scale) {
    int rc = check_kv_args(num_tokens, num_heads, head_size, num_blocks, block_size, L,
                           cache_bytes, k_scale, v_scale);
    if (rc) return rc;
    if (num_tokens == 0) return ORC_OK;
    if (!key || !value || !cache || !slot_mapping) return ORC_ERR_ARG;
    if ((rc = check_slots(slot_mapping, num_tokens, num_blocks, block_size))) return rc;
    int32_t dbytes = head_size / 2, sbytes = head_size / 16;
    uint8_t* data = (uint8_t*)malloc((size_t)dbytes);
    uint8_t* scales = (uint8_t*)malloc((size_t)sbytes);
    if (!data || !scales) { free(data); free(scales); return ORC_ERR_ARG; }
    /* Pass 0 validates every token (finite inputs, finite reciprocals);
     * pass 1 writes.  Nothing is written when pass 0 fails. */
    for (int pass = 0; pass < 2 && rc == ORC_OK; pass++) {
        for (int64_t t = 0; t < num_tokens && rc == ORC_OK; t++) {
            int64_t slot = slot_mapping[t];
            if (slot < 0) continue;                               /* padding token */
            int64_t blk = slot / block_size, off = slot % block_size;
            for (int side = 0; side < 2 && rc == ORC_OK; side++) {
                const uint16_t* src = side ? value : key;
                int64_t ts = side ? value_token_stride : key_token_stride;
                int64_t hs = side ? value_head_stride : key_head_stride;
                float gs = side ? v_scale : k_scale;
                int64_t base = blk * L->block_stride + side * L->side_stride;
                for (int32_t h = 0; h < num_heads && rc == ORC_OK; h++) {
                    const uint16_t* x = src + t * ts + h * hs;
                    for (int32_t i = 0; i < head_size; i++)
                        if (!bf16_is_finite(x[i])) rc = ORC_ERR_NONFINITE;
                    if (rc) break;
                    rc = quantize_kv_head(x, head_size, gs, data, scales);
                    if (rc || pass == 0) continue;
                    memcpy(cache + base + L->data_offset + off * L->data_token_stride
                           + h * L->data_head_stride, data, (size_t)dbytes);
                    memcpy(cache + base + L->scale_offset + off * L->scale_token_stride
                           + h * L->scale_head_stride, scales, (size_t)sbytes);
                }
            }
        }
    }
    free(data);
    free(scales);
    return rc;
}

int orc_gather_upconvert_nvfp4_kv(const uint8_t* cache, int64_t cache_bytes,
                                  uint16_t* key_out, uint16_t* value_out,
                                  int64_t total_tokens,
                                  int64_t key_token_stride, int64_t key_head_stride,
                                  int64_t value_token_stride, int64_t value_head_stride,
                                  const int32_t* block_table, int64_t block_table_stride,
                                  const int32_t* workspace_starts, const int32_t* seq_starts,
                                  int32_t batch_size, int32_t num_heads, int32_t head_size,
                                  int64_t num_blocks, int32_t block_size,
                                  const orc_kv_layout* L, float k_scale, float v_scale) {
    int rc = check_kv_args(total_tokens, num_heads, head_size, num_blocks, block_size, L,
                           cache_bytes, k_scale, v_scale);
    if (rc) return rc;
    if (total_tokens == 0) return ORC_OK;
    if (!cache || !key_out || !value_out) return ORC_ERR_ARG;
    rc = check_walk_args(total_tokens, block_table, block_table_stride, workspace_starts,
                         batch_size, block_size);
    if (rc) return rc;
    for (int64_t r = 0; r < total_tokens; r++) {               /* validate the walk */
        int64_t blk, off;
        rc = walk_row(r, block_table, block_table_stride, workspace_starts, seq_starts,
                      batch_size, num_blocks, block_size, &blk, &off);
        if (rc) return rc;
    }
    for (int64_t r = 0; r < total_tokens; r++) {
        int64_t blk, off;
        walk_row(r, block_table, block_table_stride, workspace_starts, seq_starts, batch_size,
                 num_blocks, block_size, &blk, &off);
        for (int side = 0; side < 2; side++) {
            uint16_t* out = side ? value_out : key_out;
            int64_t ts = side ? value_token_stride : key_token_stride;
            int64_t hs = side ? value_head_stride : key_head_stride;
            float gs = side ? v_scale : k_scale;
            int64_t base = blk * L->block_stride + side * L->side_stride;
            for (int32_t h = 0; h < num_heads; h++) {
                const uint8_t* data = cache + base + L->data_offset + off * L->data_token_stride
                                      + h * L->data_head_stride;
                const uint8_t* scales = cache + base + L->scale_offset
                                        + off * L->scale_token_stride + h * L->scale_head_stride;
                uint16_t* o = out + r * ts + h * hs;
                for (int32_t i = 0; i < head_size; i++) {
                    uint8_t nib = (i % 2 == 0) ? (data[i / 2] & 0xF) : (data[i / 2] >> 4);
                    float code_times_scale = orc_e2m1_decode(nib) * orc_e4m3_decode(scales[i / 16]);
                    o[i] = orc_f32_to_bf16_rne(code_times_scale * gs);
                }
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Chunked context (vLLM PR #48642 digest, the _compute_prefill_context      */
/* excerpt): chunk i gathers, for every request, the context positions that  */
/* fall in chunk i, into workspace rows laid out request after request.      */
/* READING: chunk_rows is the largest multiple of block_size such that       */
/* batch_size * chunk_rows <= workspace_rows (at most INT32_MAX); position p */
/* of a request belongs to chunk p / chunk_rows; chunk i starts every        */
/* request at position i * chunk_rows.                                       */
/* ------------------------------------------------------------------------ */
int orc_context_chunk_plan(const int32_t* context_lens, int32_t batch_size,
                           int64_t workspace_rows, int32_t block_size,
                           int32_t* chunk_rows, int32_t* num_chunks) {
    if (!context_lens || batch_size <= 0 || block_size <= 0 || workspace_rows < 0)
        return ORC_ERR_ARG;
    int64_t limit = workspace_rows < INT32_MAX ? workspace_rows : INT32_MAX;
    int64_t c = 0;                                  /* grow one block at a time */
    while ((c + block_size) * (int64_t)batch_size <= limit) c += block_size;
    if (c == 0) return ORC_ERR_ARG;
    int32_t chunks = 0;
    for (int32_t b = 0; b < batch_size; b++) {
        if (context_lens[b] < 0) return ORC_ERR_ARG;
        for (int64_t p = 0; p < context_lens[b]; p += c)   /* chunks this request touches */
            if (p / c + 1 > chunks) chunks = (int32_t)(p / c + 1);
    }
    *chunk_rows = (int32_t)c;
    *num_chunks = chunks;
    return ORC_OK;
}

int orc_context_chunk(const int32_t* context_lens, int32_t batch_size, int32_t chunk_rows,
                      int32_t chunk, int32_t* seq_starts, int32_t* workspace_starts,
                      int64_t* total_rows) {
    if (!context_lens || batch_size <= 0 || chunk_rows <= 0 || chunk < 0) return ORC_ERR_ARG;
    int64_t rows = 0;
    for (int32_t b = 0; b < batch_size; b++) {
        workspace_starts[b] = (int32_t)rows;
        seq_starts[b] = (int32_t)((int64_t)chunk * chunk_rows);
        for (int64_t p = 0; p < context_lens[b]; p++)        /* count the chunk's positions */
            if (p / chunk_rows == chunk) rows++;
    }
    *total_rows = rows;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Sparse index conversion (vLLM PR #48642 digest, "Implementation           */
/* breakdown" item 1): token row t's top-k positions, local to request       */
/* req_id[t], become global slot ids through that request's block table.    */
/* The call is rejected when req_id and token_indices differ in length.      */
/* READING: -1 for a negative position, a request id outside [0, batch), a  */
/* position past the block-table row or a block id outside the cache.       */
/* ------------------------------------------------------------------------ */
int orc_convert_req_index(const int32_t* req_id, int64_t num_req_id,
                          const int32_t* token_indices, int64_t num_tokens, int32_t topk,
                          int64_t token_indices_stride, const int32_t* block_table,
                          int32_t batch_size, int64_t block_table_stride, int32_t block_size,
                          int64_t num_blocks, int32_t* out, int64_t out_stride) {
    if (num_req_id != num_tokens) return ORC_ERR_ARG;
    if (num_tokens < 0 || topk < 0 || block_size <= 0 || batch_size <= 0 ||
        block_table_stride <= 0 || token_indices_stride < topk || out_stride < topk)
        return ORC_ERR_ARG;
    for (int64_t t = 0; t < num_tokens; t++) {
        for (int32_t k = 0; k < topk; k++) {
            int32_t i = token_indices[t * token_indices_stride + k];
            int32_t r = req_id[t];
            int64_t result = -1;
            if (i >= 0 && r >= 0 && r < batch_size && i / block_size < block_table_stride) {
                int64_t blk = block_table[(int64_t)r * block_table_stride + i / block_size];
                if (blk >= 0 && blk < num_blocks) result = blk * block_size + i % block_size;
            }
            out[t * out_stride + k] = (int32_t)result;
        }
    }
    return ORC_OK;
}
