// nvfp4_kv_kernels.hip -- gfx950 kernels for the per-head NVFP4 K/V cache
// (vLLM PR #37332 digest: "Motivation", "Implementation breakdown" item 4,
// "Key source excerpts").  The cache geometry comes in as byte offsets and
// strides (KvLayout), so the split layout, row-interleaved [data | scales]
// rows and NHD/HND orders all use the same kernels.
//
// Mapping (HBM-bound, no contraction):
//   write  : one wave per (token, side); one lane per 16-value block of a
//            head (32 B in, 8 B data + 1 scale byte out).  With 8 heads of
//            128 values a (token, side) is exactly 64 blocks = one wave.
//   gather : one wave per (row, side); one lane per 8 values (4 data bytes
//            in, 16 B bf16 out); the row's cache address is resolved once
//            per wave (wave-uniform walk).
#include "gcache_internal.h"

namespace gcache {

__device__ __forceinline__ void split_pow2(int v, int shift, int n, int& q, int& r) {
    if (shift >= 0) {
        q = v >> shift;
        r = v & (n - 1);
    } else {
        q = v / n;
        r = v - q * n;
    }
}

__global__ __launch_bounds__(kBlockThreads) void k_reshape_and_cache_nvfp4(KvWriteParams p) {
    const int lane = lane_id();
    const int bph = p.head_size >> 4;                    // 16-value blocks per head
    const int nblk = p.num_heads * bph;
    const int64_t nwork = 2 * p.num_tokens;
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave_id(); w < nwork; w += step) {
        const int64_t t = w >> 1;
        const int side = (int)(w & 1);
        const int64_t slot = p.slots[t];
        if (slot < 0) continue;                           // padding token (wave-uniform)
        int64_t blk, off;
        split_block(slot, p.div, blk, off);
        const float gs = *p.gscale[side];
        const uint16_t* x0 = p.src[side] + t * p.token_stride[side];
        uint8_t* base = p.cache + blk * p.L.block_stride + side * p.L.side_stride;
        uint8_t* data0 = base + p.L.data_offset + off * p.L.data_token_stride;
        uint8_t* scale0 = base + p.L.scale_offset + off * p.L.scale_token_stride;

        for (int b = lane; b < nblk; b += kWave) {
            int h, j;
            split_pow2(b, p.bph_shift, bph, h, j);
            const uint4* src = reinterpret_cast<const uint4*>(x0 + h * p.head_stride[side] + 16 * j);
            const uint4 v0 = src[0], v1 = src[1];
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            float x[16];
#pragma unroll
            for (int k = 0; k < 8; k++) {
                x[2 * k] = bf16_lo(wv[k]);
                x[2 * k + 1] = bf16_hi(wv[k]);
            }
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; k++) amax = fmaxf(amax, fabsf(x[k]));
            // sf = e4m3_rn_sat((amax / 6) / gs); effective scale e = dec(sf) * gs
            const uint32_t sf = put_e4m3x2<false>(0u, (amax / 6.0f) / gs, 0.0f) & 0xFFu;
            const float e = e4m3_f32(sf) * gs;
            const float inv = (e == 0.0f) ? 0.0f : 1.0f / e;
            uint32_t q0 = 0, q1 = 0;
            q0 = put_e2m1x2<0>(q0, x[0] * inv, x[1] * inv);
            q0 = put_e2m1x2<1>(q0, x[2] * inv, x[3] * inv);
            q0 = put_e2m1x2<2>(q0, x[4] * inv, x[5] * inv);
            q0 = put_e2m1x2<3>(q0, x[6] * inv, x[7] * inv);
            q1 = put_e2m1x2<0>(q1, x[8] * inv, x[9] * inv);
            q1 = put_e2m1x2<1>(q1, x[10] * inv, x[11] * inv);
            q1 = put_e2m1x2<2>(q1, x[12] * inv, x[13] * inv);
            q1 = put_e2m1x2<3>(q1, x[14] * inv, x[15] * inv);
            *reinterpret_cast<uint2*>(data0 + h * p.L.data_head_stride + 8 * j) = make_uint2(q0, q1);
            scale0[h * p.L.scale_head_stride + j] = (uint8_t)sf;
        }
    }
}

__global__ __launch_bounds__(kBlockThreads) void k_gather_nvfp4_kv(KvGatherParams p) {
    const int lane = lane_id();
    const int cph = p.head_size >> 3;                    // 8-value chunks per head
    const int nchunk = p.num_heads * cph;
    const int64_t nwork = 2 * p.total;
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave_id(); w < nwork; w += step) {
        const int64_t r = w >> 1;
        const int side = (int)(w & 1);
        const int b = find_request(p.ws, p.batch, r);
        const int64_t pos = (p.seq_starts ? (int64_t)p.seq_starts[b] : 0) + (r - (int64_t)p.ws[b]);
        int64_t bi, off;
        split_block(pos, p.div, bi, off);
        const int64_t blk = p.block_table[(int64_t)b * p.bt_stride + bi];
        const float gs = *p.gscale[side];
        const uint8_t* base = p.cache + blk * p.L.block_stride + side * p.L.side_stride;
        const uint8_t* data0 = base + p.L.data_offset + off * p.L.data_token_stride;
        const uint8_t* scale0 = base + p.L.scale_offset + off * p.L.scale_token_stride;
        uint16_t* out0 = p.out[side] + r * p.token_stride[side];

        for (int c = lane; c < nchunk; c += kWave) {
            int h, i;
            split_pow2(c, p.cph_shift, cph, h, i);       // values 8i .. 8i+7 of head h
            const uint32_t nib = *reinterpret_cast<const uint32_t*>(data0 + h * p.L.data_head_stride + 4 * i);
            const float s = e4m3_f32(scale0[h * p.L.scale_head_stride + (i >> 1)]);
            const f32x2 a = e2m1x2_f32<0>(nib), bb = e2m1x2_f32<1>(nib);
            const f32x2 cc = e2m1x2_f32<2>(nib), d = e2m1x2_f32<3>(nib);
            // (e2m1 * e4m3) is exact; one rounding for * gs, one for bf16.
            const uint4 o = make_uint4(pack_bf16x2((a.x * s) * gs, (a.y * s) * gs),
                                       pack_bf16x2((bb.x * s) * gs, (bb.y * s) * gs),
                                       pack_bf16x2((cc.x * s) * gs, (cc.y * s) * gs),
                                       pack_bf16x2((d.x * s) * gs, (d.y * s) * gs));
            *reinterpret_cast<uint4*>(out0 + h * p.head_stride[side] + 8 * i) = o;
        }
    }
}

hipError_t launch_reshape_and_cache_nvfp4(const KvWriteParams& p, hipStream_t s) {
    return launch1(k_reshape_and_cache_nvfp4, grid_for_waves(2 * p.num_tokens), s, p);
}
hipError_t launch_gather_nvfp4_kv(const KvGatherParams& p, hipStream_t s) {
    return launch1(k_gather_nvfp4_kv, grid_for_waves(2 * p.total), s, p);
}

}  // namespace gcache
