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
// reads hit in cache).  One wave per 256 indices of one token row: the row's
// request id and block-table row are wave-uniform, each lane converts 4
// consecutive indices with one 16-byte load and one 16-byte store when the
// row is 16-byte aligned, element by element otherwise.
#include "gcache_internal.h"

namespace gcache {

constexpr int kIdxPerLane = 4;
constexpr int kIdxPerWave = kIdxPerLane * kWave;

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

__global__ __launch_bounds__(kBlockThreads) void k_convert_req_index(SparseIndexParams p, int64_t wave0) {
    const int lane = lane_id();
    const int64_t w = wave0 + (int64_t)blockIdx.x * kWavesPerBlock + wave_id();
    const int64_t t = w / p.waves_per_row;
    if (t >= p.num_tokens) return;
    const int k0 = (int)(w - t * p.waves_per_row) * kIdxPerWave + kIdxPerLane * lane;
    const int32_t req = p.req_id[t];                     // wave-uniform
    const bool req_ok = req >= 0 && req < p.batch;
    const int32_t* bt_row = p.block_table + (req_ok ? (int64_t)req * p.bt_stride : 0);
    const int32_t* src = p.token_indices + t * p.ti_stride;
    int32_t* dst = p.out + t * p.out_stride;
    if (p.vec16) {                                       // topk % 4 == 0, rows 16-byte aligned
        if (k0 >= p.topk) return;
        const uint4 v = ld_stream16(src + k0);
        const uint4 o = make_uint4((uint32_t)global_slot((int32_t)v.x, bt_row, req_ok, p),
                                   (uint32_t)global_slot((int32_t)v.y, bt_row, req_ok, p),
                                   (uint32_t)global_slot((int32_t)v.z, bt_row, req_ok, p),
                                   (uint32_t)global_slot((int32_t)v.w, bt_row, req_ok, p));
        st_stream16(dst + k0, o);
    } else {
#pragma unroll
        for (int j = 0; j < kIdxPerLane; j++)
            if (k0 + j < p.topk) dst[k0 + j] = global_slot(src[k0 + j], bt_row, req_ok, p);
    }
}

hipError_t launch_convert_req_index(const SparseIndexParams& p, hipStream_t s) {
    return launch_waves(k_convert_req_index, p.num_tokens * p.waves_per_row, s, p);
}

}  // namespace gcache
