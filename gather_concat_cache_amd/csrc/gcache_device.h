// gcache_device.h -- device helpers shared by the gfx950 kernels.
//
// Conversions use the gfx950 hardware converters.  Each one is checked
// exhaustively against the CPU reference's round-to-nearest-even encoders
// over every non-NaN binary32 input (scale operand 1.0) by the GPU test
// tests/test_gpu_converters.py, which runs these helpers:
//   v_cvt_scalef32_pk_fp4_f32  e2m1, RN-even, saturating at +-6, sign kept
//                              (-0 and tiny negatives give 0x8); the first
//                              operand lands in the low nibble.
//   v_cvt_pk_fp8_f32           OCP e4m3, RN-even, sign kept; it does NOT
//                              saturate (NaN above 464), so inputs are
//                              clamped to +-448 with v_med3_f32 first, which
//                              keeps -0 and denormals.
//   v_cvt_pk_bf16_f32          RN-even (used for the rounding f32 -> bf16).
//   v_cvt_scalef32_pk_f32_fp4, v_cvt_pk_f32_fp8: exact decoders.
// The scale operand of the scalef32 forms only carries a power of two (its
// exponent field), so it is always 1.0 here and block scales are applied
// with ordinary binary32 multiplies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gcache {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;                 // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlockThreads / kWave;

// DS-MLA geometry: [vLLM PR #51724 digest, "Implementation breakdown" 2-3].
constexpr int kNope = 512;
constexpr int kRope = 64;
constexpr int kRow = kNope + kRope;                // gathered workspace row
constexpr int kNvEntry = 352;
constexpr int kNvRopeOff = 256;
constexpr int kNvScaleOff = 320;
constexpr int kF8Entry = 656;
constexpr int kF8ScaleOff = 512;
constexpr int kF8RopeOff = 528;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
// Wave index inside the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// bf16 pair in one dword -> binary32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two values -> e2m1 codes packed into byte SEL of `old` (lo -> low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t put_e2m1x2(uint32_t old, float lo, float hi) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, SEL);
}

__device__ __forceinline__ float clamp_e4m3(float v) {
    return __builtin_amdgcn_fmed3f(v, 448.0f, -448.0f);
}
// Two values -> e4m3 codes in 16-bit word HI of `old` (lo -> lower byte).
template <bool HI>
__device__ __forceinline__ uint32_t put_e4m3x2(uint32_t old, float lo, float hi) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(lo), clamp_e4m3(hi), (int)old, HI);
}

// Byte SEL of `packed` (two e2m1 codes) -> two binary32 (exact).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t packed) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
}
// Word HI of `packed` (two e4m3 codes) -> two binary32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t packed) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)packed, HI);
}
// Low byte of `b` (one e4m3 code) -> binary32 (exact).
__device__ __forceinline__ float e4m3_f32(uint32_t b) { return e4m3x2_f32<false>(b).x; }

// Two binary32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Streaming accesses.  Every input byte of these kernels is read once and
// every output byte written once, so loads and stores carry the nontemporal
// hint: in the dirty-cache state a pipeline of such ops runs in, this keeps
// the streams from evicting (and writing back) lines in the 256 MB
// last-level cache and L2, which measured +15-25% on the gathers and the
// writes.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_stream4(const void* p) {
    return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t ld_stream1(const void* p) {
    return __builtin_nontemporal_load(static_cast<const uint8_t*>(p));
}
// The 16-byte store every kernel writes its outputs with also carries the
// system-scope bits (sc0 sc1): the piece is written through to memory
// instead of staying dirty in L2, so a kernel leaves no write-back for the
// next one on the stream to absorb (measured in the six-op pass: the writes
// and the fp8 gather 1-2 % faster, the metric's pair +1-1.5 %).  No builtin
// sets these bits on a global store, hence one global_store_dwordx4 in
// inline asm (a vector store); the s_nop keeps two wait states before a
// VALU may overwrite the store's data registers.
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\ts_nop 1" : : "v"(p), "v"(w) : "memory");
}
__device__ __forceinline__ void st_stream8(void* p, uint2 v) {
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, static_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_stream4(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, static_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_stream2(void* p, uint16_t v) {
    __builtin_nontemporal_store(v, static_cast<uint16_t*>(p));
}
__device__ __forceinline__ void st_stream1(void* p, uint8_t v) {
    __builtin_nontemporal_store(v, static_cast<uint8_t*>(p));
}

// Split a slot (or logical position) into (block, offset).  `shift` >= 0
// when block_size is a power of two.
// A slot id outside [0, num_slots) -- padding (-1) or out of range -- is
// skipped: it becomes -1.
__device__ __forceinline__ int64_t valid_slot(int64_t slot, int64_t num_slots) {
    return (uint64_t)slot < (uint64_t)num_slots ? slot : -1;
}

struct BlockDiv {
    int64_t size;
    int shift;
};
__host__ __device__ __forceinline__ void split_block(int64_t pos, const BlockDiv& d, int64_t& blk,
                                                     int64_t& off) {
    if (d.shift >= 0) {
        blk = pos >> d.shift;
        off = pos & (d.size - 1);
    } else {
        blk = pos / d.size;
        off = pos - blk * d.size;
    }
}

// Gather walk: request of workspace row r = the largest b < batch with
// ws[b] <= r (ws non-decreasing, ws[0] == 0).  The search starts at the
// interpolated guess r * batch / total and gallops outwards, then bisects the
// bracket: about two probes when requests are evenly sized (one row per
// request, for instance) and at most about twice a plain bisection.
__host__ __device__ __forceinline__ int find_request(const int32_t* __restrict__ ws, int batch, int64_t r,
                                           int64_t total) {
    int lo, hi;                                    // invariant: ws[lo] <= r < ws[hi] (hi == batch: +inf)
    int g = (int)((r * (int64_t)batch) / total);
    if (g >= batch) g = batch - 1;
    if ((int64_t)ws[g] <= r) {
        lo = g;
        int step = 1;
        hi = g + 1;
        while (hi < batch && (int64_t)ws[hi] <= r) {
            lo = hi;
            step <<= 1;
            hi = (lo + step < batch) ? lo + step : batch;
        }
    } else {
        hi = g;
        int step = 1;
        lo = g > 0 ? g - 1 : 0;
        while (lo > 0 && (int64_t)ws[lo] > r) {
            hi = lo;
            step <<= 1;
            lo = (hi - step > 0) ? hi - step : 0;
        }
        // Stopping at lo == 0 with ws[0] > r happens only when ws[0] != 0
        // (invalid input): the result is then some request in [0, batch).
    }
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)ws[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

// The same search for batch <= 64 as a fixed six-step bisection, so that all
// lanes of a wave run identical steps; ws_at(i) returns ws[i] (on the device
// a cross-lane read of the lane that holds it).  Returns the largest b in
// [0, batch) with ws[b] <= r for non-decreasing ws with ws[0] == 0, and some
// b in [0, batch) for any other ws.
template <typename WsAt>
__host__ __device__ __forceinline__ int bisect_request64(WsAt ws_at, int batch, int64_t r) {
    int lo = 0, hi = batch;                        // lo <= mid < hi <= batch
#pragma unroll
    for (int it = 0; it < 6; it++) {
        const int mid = (lo + hi) >> 1;
        const int64_t wm = ws_at(mid);
        if (hi - lo > 1) {
            if (wm <= r) lo = mid;
            else hi = mid;
        }
    }
    return lo;
}

// Cache byte offset of the entry read by workspace row r of request b, or -1
// when the row's position falls outside [0, bt_stride * block_size) or its
// block id outside [0, num_blocks) (the kernels then write a zero row).
__host__ __device__ __forceinline__ int64_t row_entry(const int32_t* __restrict__ block_table,
                                                      int64_t bt_stride, int b, int64_t ws_b,
                                                      int64_t seq_start_b, int64_t r,
                                                      const BlockDiv& div, int64_t num_blocks,
                                                      int64_t block_stride, int64_t entry_stride) {
    const int64_t pos = seq_start_b + (r - ws_b);
    if (pos < 0) return -1;
    int64_t bi, off;
    split_block(pos, div, bi, off);
    if (bi >= bt_stride) return -1;
    const int64_t blk = block_table[(int64_t)b * bt_stride + bi];
    if (blk < 0 || blk >= num_blocks) return -1;
    return blk * block_stride + off * entry_stride;
}

}  // namespace gcache
