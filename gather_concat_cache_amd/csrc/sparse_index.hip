// sparse_index.hip -- request-local top-k token indices -> global cache slot
// ids for the sparse decode path (vLLM PR #48642 digest, "Implementation
// breakdown" item 1: the conversion rejects a req_id / token_indices length
// mismatch instead of running its grid past the smaller one).
//
// out[t, k] = block_table[req_id[t], i / block_size] * block_size + i % block_size
// for i = token_indices[t, k]; -1 when i < 0, the request id is outside
// [0, batch), i / block_size is outside the block-table row, or the block id
// is outside [0, num_blocks).
//
// Mapping: HBM-bound (4 bytes in, 4 bytes out per index; the block-table
// reads hit in cache).  Each wave takes a run of one token row, so the row's
// request id and block-table row are wave-uniform.  When the rows are
// 16-byte aligned (topk % 4 == 0) a wave converts 1024 indices: each lane
// issues four 16-byte loads of 4 indices (consecutive lanes on consecutive
// pieces, all in flight) and four 16-byte stores, which keeps enough bytes
// in flight that the whole 4096 x 2048 conversion runs in about one round
// of resident waves; otherwise a wave converts 256 indices element by
// element.
#include "gcache_internal.h"

namespace gcache {

constexpr int kIdxPerLane = 4;                          // element path
constexpr int kIdxPerWave = kIdxPerLane * kWave;         // 256
constexpr int kPiecesPerLane = 4;                        // 16-byte path: 4 x 4 indices per lane
constexpr int kIdxPerWaveVec = 4 * kPiecesPerLane * kWave;   // 1024

__device__ __forceinline__ int32_t global_slot(int32_t i, const int32_t* __restrict__ bt_row, bool req_ok,
                                               const SparseIndexParams& p) {
    if (!req_ok || i < 0) return -1;
    int64_t bi, off;
    split_block(i, p.div, bi, off);
    if (bi >= p.bt_stride) return -1;
    const int32_t blk = bt_row[bi];
    if (blk < 0 || blk >= p.num_blocks) return -1;
    return (int32_t)(blk * p.div.size + off);
}

template <bool VEC16>
__global__ __launch_bounds__(kBlockThreads) void k_convert_req_index(SparseIndexParams p, int64_t wave0) {
    const int lane = lane_id();
    const int64_t w = wave0 + (int64_t)blockIdx.x * kWavesPerBlock + wave_id();
    const int64_t t = w / p.waves_per_row;
    if (t >= p.num_tokens) return;
    const int run = (int)(w - t * p.waves_per_row);
    const int32_t req = p.req_id[t];                     // wave-uniform
    const bool req_ok = req >= 0 && req < p.batch;
    const int32_t* bt_row = p.block_table + (req_ok ? (int64_t)req * p.bt_stride : 0);
    const int32_t* src = p.token_indices + t * p.ti_stride;
    int32_t* dst = p.out + t * p.out_stride;
    if (VEC16) {                                         // topk % 4 == 0, rows 16-byte aligned
        const int kbase = run * kIdxPerWaveVec;
        uint4 v[kPiecesPerLane];
#pragma unroll
        for (int j = 0; j < kPiecesPerLane; j++) {       // all loads first
            const int k = kbase + 4 * (lane + kWave * j);
            if (k < p.topk) v[j] = ld_stream16(src + k);
        }
#pragma unroll
        for (int j = 0; j < kPiecesPerLane; j++) {
            const int k = kbase + 4 * (lane + kWave * j);
            if (k >= p.topk) continue;
            const uint4 o = make_uint4((uint32_t)global_slot((int32_t)v[j].x, bt_row, req_ok, p),
                                       (uint32_t)global_slot((int32_t)v[j].y, bt_row, req_ok, p),
                                       (uint32_t)global_slot((int32_t)v[j].z, bt_row, req_ok, p),
                                       (uint32_t)global_slot((int32_t)v[j].w, bt_row, req_ok, p));
            st_stream16(dst + k, o);
        }
    } else {
        const int k0 = run * kIdxPerWave + kIdxPerLane * lane;
#pragma unroll
        for (int j = 0; j < kIdxPerLane; j++)
            if (k0 + j < p.topk) dst[k0 + j] = global_slot(src[k0 + j], bt_row, req_ok, p);
    }
}

hipError_t launch_convert_req_index(const SparseIndexParams& p, hipStream_t s) {
    SparseIndexParams q = p;
    const int per_wave = q.vec16 ? kIdxPerWaveVec : kIdxPerWave;
    q.waves_per_row = (q.topk + per_wave - 1) / per_wave;
    return q.vec16 ? launch_waves(k_convert_req_index<true>, q.num_tokens * q.waves_per_row, s, q)
                   : launch_waves(k_convert_req_index<false>, q.num_tokens * q.waves_per_row, s, q);
}

}  // namespace gcache
