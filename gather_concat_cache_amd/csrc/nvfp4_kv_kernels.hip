// nvfp4_kv_kernels.hip -- gfx950 kernels for the per-head NVFP4 K/V cache
// (vLLM PR #37332 digest: "Motivation", "Implementation breakdown" item 4,
// "Key source excerpts").  The cache geometry comes in as byte offsets and
// strides (KvLayout), so the split layout, row-interleaved [data | scales]
// rows and NHD/HND orders all use the same kernels.
//
// Mapping (HBM-bound, no contraction; streaming loads and stores):
//   write  : one-shot wave per token; one lane per 16-value block of a head and
//            side (32 B in, 8 B data + 1 scale byte out).  With 8 heads of
//            128 values a side is exactly 64 blocks, so both sides' loads
//            (64 B per lane) are in flight before any is used.
//   staged : when each (token, side) of the layout is at most two
//            contiguous, 16-byte aligned runs -- the token's data of all
//            heads and its scales of all heads (the NHD split layout), or
//            one run of [data | scales] rows (the interleaved-row
//            arrangement) -- the write assembles the runs in LDS and stores
//            16-byte pieces, and the gather loads them as 16-byte pieces
//            into LDS first.
//   gather : one workspace row per one-shot wave (both sides, all heads);
//            the row's cache address is resolved once (wave-uniform search
//            over workspace_starts, one block-table load), then one lane per
//            8 values (4 data bytes in, 16 B bf16 out), every load of a pass
//            issued before any conversion.
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

constexpr int kKvItemsPerLane = 2;   // blocks in flight per lane and pass
constexpr int kKvMaxSpan = 2048;     // largest staged (token, side) run, bytes

// Cache byte offset of byte b of a staged (token, side) image: image bytes
// [0, run0) are run 0 (the data run), the rest run 1 (the scale run).
__device__ __forceinline__ int64_t kv_run_offset(const KvLayout& L, const KvStage& st, int64_t blk, int side,
                                                 int64_t off, int b) {
    const int64_t base = blk * L.block_stride + side * L.side_stride;
    return b < st.run0 ? base + L.data_offset + off * L.data_token_stride + b
                       : base + L.scale_offset + off * L.scale_token_stride + (b - st.run0);
}

// STAGED: the layout keeps each (token, side) in at most two contiguous,
// 16-byte aligned runs (see staged_layout).  The wave then assembles the
// token's images in LDS and writes them as 16-byte pieces instead of 8-byte
// code runs and single scale bytes that each cover part of a line.
template <bool STAGED>
__global__ __launch_bounds__(kBlockThreads) void k_reshape_and_cache_nvfp4(KvWriteParams p, int64_t wave0) {
    __shared__ __align__(16) uint8_t s_img[STAGED ? kWavesPerBlock : 1][STAGED ? 2 * kKvMaxSpan : 16];
    const int lane = lane_id();
    const int bph = p.head_size >> 4;                    // 16-value blocks per head
    const int nblk = p.num_heads * bph;                  // per side
    const int nitems = 2 * nblk;                         // both sides
    const int64_t t = wave0 + (int64_t)blockIdx.x * kWavesPerBlock + wave_id();
    if (t >= p.num_tokens) return;
    {
        // The slot, the scales and the first pass of inputs are loaded
        // together (a skipped token's inputs are read but never used).
        const int64_t slot_in = p.slots[t];
        const float gs_k = *p.gscale[0], gs_v = *p.gscale[1];
        int64_t slot = -1, blk = 0, off = 0;

        for (int base = 0; base < nitems; base += kKvItemsPerLane * kWave) {
            uint4 v0[kKvItemsPerLane], v1[kKvItemsPerLane];
#pragma unroll
            for (int u = 0; u < kKvItemsPerLane; u++) {
                const int it = base + u * kWave + lane;
                if (it < nitems) {
                    const int side = it >= nblk;
                    int h, j;
                    split_pow2(it - side * nblk, p.bph_shift, bph, h, j);
                    const uint8_t* src = reinterpret_cast<const uint8_t*>(
                        p.src[side] + t * p.token_stride[side] + h * p.head_stride[side] + 16 * j);
                    v0[u] = ld_stream16(src);
                    v1[u] = ld_stream16(src + 16);
                }
            }
            if (base == 0) {
                slot = valid_slot(slot_in, p.num_slots);
                if (slot < 0) return;                     // skipped token (wave-uniform)
                split_block(slot, p.div, blk, off);
            }
#pragma unroll
            for (int u = 0; u < kKvItemsPerLane; u++) {
                const int it = base + u * kWave + lane;
                if (it >= nitems) continue;
                const int side = it >= nblk;
                int h, j;
                split_pow2(it - side * nblk, p.bph_shift, bph, h, j);
                const float gs = side ? gs_v : gs_k;
                const uint32_t wv[8] = {v0[u].x, v0[u].y, v0[u].z, v0[u].w,
                                        v1[u].x, v1[u].y, v1[u].z, v1[u].w};
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
                if (STAGED) {                            // image of the token's (token, side) runs
                    uint8_t* img = s_img[wave_id()] + side * p.st.span;
                    *reinterpret_cast<uint2*>(img + h * p.st.data_head + 8 * j) = make_uint2(q0, q1);
                    img[p.st.scale_off + h * p.st.scale_head + j] = (uint8_t)sf;
                    continue;
                }
                uint8_t* base_ptr = p.cache + blk * p.L.block_stride + side * p.L.side_stride;
                st_stream8(base_ptr + p.L.data_offset + off * p.L.data_token_stride
                               + h * p.L.data_head_stride + 8 * j,
                           make_uint2(q0, q1));
                st_stream1(base_ptr + p.L.scale_offset + off * p.L.scale_token_stride
                               + h * p.L.scale_head_stride + j,
                           (uint8_t)sf);
            }
        }
        if (STAGED) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint8_t* img = s_img[wave_id()];
            const int pieces = p.st.span >> 4;           // per side
            for (int q = lane; q < 2 * pieces; q += kWave) {
                const int side = q >= pieces;
                const int k = q - side * pieces;
                st_stream16(p.cache + kv_run_offset(p.L, p.st, blk, side, off, 16 * k),
                            *reinterpret_cast<const uint4*>(img + side * p.st.span + 16 * k));
            }
        }
    }
}

constexpr int kKvGatherItems = 4;   // 8-value chunks per lane and pass

// STAGED: as for the write, each (token, side) is at most two contiguous
// runs; the wave loads the row's runs as 16-byte pieces into LDS and
// converts from there instead of 4-byte code and 1-byte scale loads.
template <bool STAGED>
__global__ __launch_bounds__(kBlockThreads) void k_gather_nvfp4_kv(KvGatherParams p, int64_t wave0) {
    __shared__ __align__(16) uint8_t s_img[STAGED ? kWavesPerBlock : 1][STAGED ? 2 * kKvMaxSpan : 16];
    const int lane = lane_id();
    const int cph = p.head_size >> 3;                    // 8-value chunks per head
    const int nchunk = p.num_heads * cph;                // per side
    const int nitems = 2 * nchunk;                       // both sides
    const int64_t r = wave0 + (int64_t)blockIdx.x * kWavesPerBlock + wave_id();
    if (r >= p.total) return;
    // Wave-uniform walk of row r.  The interpolated guess g and its
    // neighbour are loaded together with seq_starts[g]: when
    // ws[g] <= r < ws[g+1] the request is g and no further load is needed
    // (one request per row, or evenly sized requests); otherwise the full
    // search runs.  blk < 0: the walk leaves the block table or the cache,
    // and the row is written as zeros.
    int g = (int)((r * (int64_t)p.batch) / p.total);
    if (g >= p.batch) g = p.batch - 1;
    const int64_t ws_g = p.ws[g];
    const int64_t ws_n = g + 1 < p.batch ? (int64_t)p.ws[g + 1] : INT64_MAX;
    const int64_t ss_g = p.seq_starts ? (int64_t)p.seq_starts[g] : 0;
    int b = g;
    int64_t ws_b = ws_g, ss_b = ss_g;
    if (!(ws_g <= r && r < ws_n)) {
        b = find_request(p.ws, p.batch, r, p.total);
        ws_b = p.ws[b];
        ss_b = p.seq_starts ? (int64_t)p.seq_starts[b] : 0;
    }
    const int64_t pos = ss_b + (r - ws_b);
    int64_t bi = -1, off = 0, blk = -1;
    if (pos >= 0) split_block(pos, p.div, bi, off);
    if (bi >= 0 && bi < p.bt_stride) {
        blk = p.block_table[(int64_t)b * p.bt_stride + bi];
        if (blk >= p.num_blocks) blk = -1;
    }
    const float gs_k = *p.gscale[0], gs_v = *p.gscale[1];

    if (STAGED && blk >= 0) {                            // the row's runs -> LDS
        uint8_t* img = s_img[wave_id()];
        const int pieces = p.st.span >> 4;
        for (int q = lane; q < 2 * pieces; q += kWave) {
            const int side = q >= pieces;
            const int k = q - side * pieces;
            *reinterpret_cast<uint4*>(img + side * p.st.span + 16 * k) =
                ld_stream16(p.cache + kv_run_offset(p.L, p.st, blk, side, off, 16 * k));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    for (int base = 0; base < nitems; base += kKvGatherItems * kWave) {
        uint32_t nib[kKvGatherItems] = {}, sfb[kKvGatherItems] = {};
#pragma unroll
        for (int u = 0; u < kKvGatherItems; u++) {       // all loads of the pass first
            const int it = base + u * kWave + lane;
            if (it < nitems && blk >= 0) {
                const int side = it >= nchunk;
                int h, i;
                split_pow2(it - side * nchunk, p.cph_shift, cph, h, i);   // values 8i..8i+7 of head h
                if (STAGED) {
                    const uint8_t* img = s_img[wave_id()] + side * p.st.span;
                    nib[u] = *reinterpret_cast<const uint32_t*>(img + h * p.st.data_head + 4 * i);
                    sfb[u] = img[p.st.scale_off + h * p.st.scale_head + (i >> 1)];
                    continue;
                }
                const uint8_t* sb = p.cache + blk * p.L.block_stride + side * p.L.side_stride;
                nib[u] = ld_stream4(sb + p.L.data_offset + off * p.L.data_token_stride
                                    + h * p.L.data_head_stride + 4 * i);
                sfb[u] = ld_stream1(sb + p.L.scale_offset + off * p.L.scale_token_stride
                                    + h * p.L.scale_head_stride + (i >> 1));
            }
        }
#pragma unroll
        for (int u = 0; u < kKvGatherItems; u++) {
            const int it = base + u * kWave + lane;
            if (it >= nitems) continue;
            const int side = it >= nchunk;
            int h, i;
            split_pow2(it - side * nchunk, p.cph_shift, cph, h, i);
            const float gs = side ? gs_v : gs_k;
            const float s = e4m3_f32(sfb[u]);
            const f32x2 a = e2m1x2_f32<0>(nib[u]), bb = e2m1x2_f32<1>(nib[u]);
            const f32x2 cc = e2m1x2_f32<2>(nib[u]), d = e2m1x2_f32<3>(nib[u]);
            // (e2m1 * e4m3) is exact; one rounding for * gs, one for bf16.
            uint4 o = make_uint4(pack_bf16x2((a.x * s) * gs, (a.y * s) * gs),
                                 pack_bf16x2((bb.x * s) * gs, (bb.y * s) * gs),
                                 pack_bf16x2((cc.x * s) * gs, (cc.y * s) * gs),
                                 pack_bf16x2((d.x * s) * gs, (d.y * s) * gs));
            if (blk < 0) o = make_uint4(0, 0, 0, 0);
            st_stream16(p.out[side] + r * p.token_stride[side] + h * p.head_stride[side] + 8 * i, o);
        }
    }
}

hipError_t launch_reshape_and_cache_nvfp4(const KvWriteParams& p, hipStream_t s) {
    return p.st.span ? launch_waves(k_reshape_and_cache_nvfp4<true>, p.num_tokens, s, p)
                     : launch_waves(k_reshape_and_cache_nvfp4<false>, p.num_tokens, s, p);
}
hipError_t launch_gather_nvfp4_kv(const KvGatherParams& p, hipStream_t s) {
    return p.st.span ? launch_waves(k_gather_nvfp4_kv<true>, p.total, s, p)
                     : launch_waves(k_gather_nvfp4_kv<false>, p.total, s, p);
}

// The staged kernels apply when each (token, side) of the layout is at most
// two contiguous, 16-byte aligned runs of at most kKvMaxSpan bytes in all:
//   rows  : [data | scales] rows, head after head -- one run of H * full_dim;
//   split : the heads' data back to back (head stride head_size / 2) and the
//           heads' scales back to back (head stride head_size / 16), each
//           run a whole number of 16-byte pieces -- the NHD split layout.
// Otherwise (HND, padded heads, odd sizes) the direct kernels run.
KvStage staged_layout(const KvLayout& L, int32_t num_heads, int32_t head_size) {
    const int64_t dr = head_size / 2, sr = head_size / 16, fd = dr + sr, span = num_heads * fd;
    KvStage st{0, 0, 0, 0, 0};
    if (span > kKvMaxSpan || L.side_stride % 16 || L.block_stride % 16 || L.data_offset % 16 ||
        L.data_token_stride % 16)
        return st;
    const bool rows = L.data_head_stride == fd && L.scale_head_stride == fd && L.scale_offset == L.data_offset + dr &&
                      L.data_token_stride == span && L.scale_token_stride == span && span % 16 == 0;
    if (rows) return KvStage{(int32_t)span, (int32_t)span, (int32_t)fd, (int32_t)dr, (int32_t)fd};
    const int64_t drun = num_heads * dr, srun = num_heads * sr;
    const bool split = L.data_head_stride == dr && L.scale_head_stride == sr && drun % 16 == 0 && srun % 16 == 0 &&
                       L.scale_offset % 16 == 0 && L.scale_token_stride % 16 == 0;
    if (split) return KvStage{(int32_t)span, (int32_t)drun, (int32_t)dr, (int32_t)drun, (int32_t)sr};
    return st;
}

}  // namespace gcache
