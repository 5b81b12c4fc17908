// ds_mla_kernels.hip -- gfx950 kernels for the DS-MLA paged KV cache:
// nvfp4_ds_mla and fp8_ds_mla write, and their gather-upconvert into a
// contiguous bf16 [rows, 576] workspace.
//
// Formats: vLLM PR #51724 digest ("Implementation breakdown" items 2-3, the
// kernel excerpts under "Key source excerpts"); the gather walk with
// seq_starts: vLLM PR #48642 digest ("Implementation breakdown" item 2).
//
// All four kernels are HBM-bound streams with no contraction.  Mapping:
//   nvfp4 write : one lane per 16-value NoPE block (32 B in, 8 B + 1 scale
//                 byte out), so a wave covers two tokens and needs no
//                 cross-lane reduction; the block's amax, scale and
//                 reciprocal are computed once per lane.
//   fp8 write   : one wave per token, 8 values per lane (one 16 B load);
//                 the 128-value group amax is a 4-step DPP butterfly inside
//                 each 16-lane row.
//   gathers     : one wave per 16 workspace rows; lanes 0..15 resolve the
//                 rows' cache addresses in parallel (binary search over
//                 workspace_starts, one block-table load), then every row is
//                 read and written with whole-wave contiguous accesses
//                 (NoPE: 4 or 8 B per lane in, 16 B per lane out).
#include "gcache_internal.h"

namespace gcache {

// ---------------------------------------------------------------------------
// nvfp4_ds_mla write
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void k_write_nvfp4_ds_mla(DsMlaWriteParams p) {
    const int lane = lane_id();
    const int half = lane >> 5;   // token of the pair
    const int j = lane & 31;      // NoPE block (values 16j .. 16j+15), RoPE pair j
    const int64_t npairs = (p.num_tokens + 1) >> 1;
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t pair = (int64_t)blockIdx.x * kWavesPerBlock + wave_id(); pair < npairs;
         pair += step) {
        const int64_t t = 2 * pair + half;
        if (t >= p.num_tokens) continue;
        const int64_t slot = p.slots[t];
        if (slot < 0) continue;                               // padding token

        const uint4* src = reinterpret_cast<const uint4*>(p.kv_c + t * p.kv_c_stride) + 2 * j;
        const uint4 v0 = src[0], v1 = src[1];
        const uint32_t rw = reinterpret_cast<const uint32_t*>(p.k_pe + t * p.k_pe_stride)[j];

        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float x[16];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            x[2 * k] = bf16_lo(w[k]);
            x[2 * k + 1] = bf16_hi(w[k]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; k++) amax = fmaxf(amax, fabsf(x[k]));

        // Block scale: e4m3_rn_sat(amax / 6), then the binary32 reciprocal of
        // its decoded value (0 for a zero scale).
        const uint32_t sf = put_e4m3x2<false>(0u, amax / 6.0f, 0.0f) & 0xFFu;
        const float s = e4m3_f32(sf);
        const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;

        uint32_t q0 = 0, q1 = 0;
        q0 = put_e2m1x2<0>(q0, x[0] * inv, x[1] * inv);
        q0 = put_e2m1x2<1>(q0, x[2] * inv, x[3] * inv);
        q0 = put_e2m1x2<2>(q0, x[4] * inv, x[5] * inv);
        q0 = put_e2m1x2<3>(q0, x[6] * inv, x[7] * inv);
        q1 = put_e2m1x2<0>(q1, x[8] * inv, x[9] * inv);
        q1 = put_e2m1x2<1>(q1, x[10] * inv, x[11] * inv);
        q1 = put_e2m1x2<2>(q1, x[12] * inv, x[13] * inv);
        q1 = put_e2m1x2<3>(q1, x[14] * inv, x[15] * inv);
        const uint32_t rq = put_e4m3x2<false>(0u, bf16_lo(rw), bf16_hi(rw));

        int64_t blk, off;
        split_block(slot, p.div, blk, off);
        uint8_t* e = p.cache + blk * p.block_stride + off * p.entry_stride;
        *reinterpret_cast<uint2*>(e + 8 * j) = make_uint2(q0, q1);
        *reinterpret_cast<uint16_t*>(e + kNvRopeOff + 2 * j) = (uint16_t)rq;
        e[kNvScaleOff + j] = (uint8_t)sf;
    }
}

// ---------------------------------------------------------------------------
// fp8_ds_mla write: 512 e4m3 | 4 x fp32 scale (amax / 448 per 128) | 64 bf16
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__global__ __launch_bounds__(kBlockThreads) void k_write_fp8_ds_mla(DsMlaWriteParams p) {
    const int lane = lane_id();
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave_id(); t < p.num_tokens;
         t += step) {
        const int64_t slot = p.slots[t];
        if (slot < 0) continue;                               // wave-uniform

        const uint4 v = reinterpret_cast<const uint4*>(p.kv_c + t * p.kv_c_stride)[lane];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            x[2 * k] = bf16_lo(w[k]);
            x[2 * k + 1] = bf16_hi(w[k]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) amax = fmaxf(amax, fabsf(x[k]));
        // 16 lanes x 8 values = one 128-value group: butterfly max in the row.
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));    // quad_perm [1,0,3,2]
        amax = fmaxf(amax, dpp_f32<0x4E>(amax));    // quad_perm [2,3,0,1]
        amax = fmaxf(amax, dpp_f32<0x141>(amax));   // row_half_mirror
        amax = fmaxf(amax, dpp_f32<0x140>(amax));   // row_mirror

        const float sc = amax / 448.0f;
        const float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
        uint32_t q0 = 0, q1 = 0;
        q0 = put_e4m3x2<false>(q0, x[0] * inv, x[1] * inv);
        q0 = put_e4m3x2<true>(q0, x[2] * inv, x[3] * inv);
        q1 = put_e4m3x2<false>(q1, x[4] * inv, x[5] * inv);
        q1 = put_e4m3x2<true>(q1, x[6] * inv, x[7] * inv);

        int64_t blk, off;
        split_block(slot, p.div, blk, off);
        uint8_t* e = p.cache + blk * p.block_stride + off * p.entry_stride;
        reinterpret_cast<uint2*>(e)[lane] = make_uint2(q0, q1);
        if ((lane & 15) == 0) reinterpret_cast<float*>(e + kF8ScaleOff)[lane >> 4] = sc;
        if (lane < 8) {
            const uint4 r = reinterpret_cast<const uint4*>(p.k_pe + t * p.k_pe_stride)[lane];
            reinterpret_cast<uint4*>(e + kF8RopeOff)[lane] = r;
        }
    }
}

// ---------------------------------------------------------------------------
// gathers
// ---------------------------------------------------------------------------
constexpr int kRowsPerWave = 16;

// Cache byte offset of the entry read by workspace row r.
__device__ __forceinline__ int64_t row_entry_offset(const DsMlaGatherParams& p, int64_t r) {
    const int b = find_request(p.ws, p.batch, r);
    const int64_t pos = (p.seq_starts ? (int64_t)p.seq_starts[b] : 0) + (r - (int64_t)p.ws[b]);
    int64_t bi, off;
    split_block(pos, p.div, bi, off);
    const int64_t blk = p.block_table[(int64_t)b * p.bt_stride + bi];
    return blk * p.block_stride + off * p.entry_stride;
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int k) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, k);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), k);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t shfl64(int64_t v, int src_lane) {
    const uint32_t lo = __builtin_amdgcn_ds_bpermute(src_lane << 2, (int)(uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_ds_bpermute(src_lane << 2, (int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <bool NVFP4>
__global__ __launch_bounds__(kBlockThreads) void k_gather_ds_mla(DsMlaGatherParams p) {
    const int lane = lane_id();
    const int64_t ngroups = (p.total + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t g = (int64_t)blockIdx.x * kWavesPerBlock + wave_id(); g < ngroups; g += step) {
        const int64_t r0 = g * kRowsPerWave;
        const int nrows = (int)min((int64_t)kRowsPerWave, p.total - r0);
        int64_t eoff = 0;
        if (lane < nrows) eoff = row_entry_offset(p, r0 + lane);

        // NoPE: one row per iteration, the whole wave on one entry.
#pragma unroll
        for (int k = 0; k < kRowsPerWave; k++) {
            if (k >= nrows) continue;
            const uint8_t* e = p.cache + readlane64(eoff, k);
            uint4 o;
            if (NVFP4) {
                const uint32_t nib = reinterpret_cast<const uint32_t*>(e)[lane];  // values 8l..8l+7
                const float s = e4m3_f32(e[kNvScaleOff + (lane >> 1)]);
                const f32x2 a = e2m1x2_f32<0>(nib), b = e2m1x2_f32<1>(nib);
                const f32x2 c = e2m1x2_f32<2>(nib), d = e2m1x2_f32<3>(nib);
                o = make_uint4(pack_bf16x2(a.x * s, a.y * s), pack_bf16x2(b.x * s, b.y * s),
                               pack_bf16x2(c.x * s, c.y * s), pack_bf16x2(d.x * s, d.y * s));
            } else {
                const uint2 q = reinterpret_cast<const uint2*>(e)[lane];          // codes 8l..8l+7
                const float sc = reinterpret_cast<const float*>(e + kF8ScaleOff)[lane >> 4];
                const f32x2 a = e4m3x2_f32<false>(q.x), b = e4m3x2_f32<true>(q.x);
                const f32x2 c = e4m3x2_f32<false>(q.y), d = e4m3x2_f32<true>(q.y);
                o = make_uint4(pack_bf16x2(a.x * sc, a.y * sc), pack_bf16x2(b.x * sc, b.y * sc),
                               pack_bf16x2(c.x * sc, c.y * sc), pack_bf16x2(d.x * sc, d.y * sc));
            }
            reinterpret_cast<uint4*>(p.dst + (r0 + k) * p.dst_stride)[lane] = o;
        }

        // RoPE: 8 rows per pass, 8 lanes per row, 8 values (16 B out) per lane.
#pragma unroll
        for (int h = 0; h < kRowsPerWave / 8; h++) {
            const int k = 8 * h + (lane >> 3);
            const int c = lane & 7;
            const int64_t eo = shfl64(eoff, k);
            if (k < nrows) {
                const uint8_t* e = p.cache + eo;
                uint4 o;
                if (NVFP4) {
                    const uint2 q = reinterpret_cast<const uint2*>(e + kNvRopeOff)[c];
                    const f32x2 a = e4m3x2_f32<false>(q.x), b = e4m3x2_f32<true>(q.x);
                    const f32x2 cc = e4m3x2_f32<false>(q.y), d = e4m3x2_f32<true>(q.y);
                    o = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y),
                                   pack_bf16x2(cc.x, cc.y), pack_bf16x2(d.x, d.y));
                } else {
                    o = reinterpret_cast<const uint4*>(e + kF8RopeOff)[c];
                }
                reinterpret_cast<uint4*>(p.dst + (r0 + k) * p.dst_stride + kNope)[c] = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_write_nvfp4_ds_mla(const DsMlaWriteParams& p, hipStream_t s) {
    return launch1(k_write_nvfp4_ds_mla, grid_for_waves((p.num_tokens + 1) / 2), s, p);
}
hipError_t launch_write_fp8_ds_mla(const DsMlaWriteParams& p, hipStream_t s) {
    return launch1(k_write_fp8_ds_mla, grid_for_waves(p.num_tokens), s, p);
}
hipError_t launch_gather_nvfp4_ds_mla(const DsMlaGatherParams& p, hipStream_t s) {
    return launch1(k_gather_ds_mla<true>,
                   grid_for_waves((p.total + kRowsPerWave - 1) / kRowsPerWave), s, p);
}
hipError_t launch_gather_fp8_ds_mla(const DsMlaGatherParams& p, hipStream_t s) {
    return launch1(k_gather_ds_mla<false>,
                   grid_for_waves((p.total + kRowsPerWave - 1) / kRowsPerWave), s, p);
}

}  // namespace gcache
