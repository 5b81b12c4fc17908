// bench_ceiling.hip -- libgcache_bench.so: the same-mix copy that bench.py
// uses as an on-device ceiling for the cache operations (declared in
// include/gcache_bench.h).  Not part of the cache path.
#include "../../include/gcache_bench.h"
#include "gcache_device.h"

namespace {

using namespace gcache;

constexpr int kTile = 16;                       // rows per workgroup
constexpr int kMaxPieces = 72;                  // 1152 bytes per row at most
constexpr int kLoads = (kTile * kMaxPieces + kBlockThreads - 1) / kBlockThreads;

struct CopyMixParams {
    const uint8_t* src;
    uint8_t* dst;
    int64_t rows;
    int32_t rp, wp;                             // 16-byte pieces read / written per row
};

// One workgroup per 16 rows: every input piece of the tile is loaded (all
// loads in flight), staged in LDS, then the output pieces are stored.
__global__ __launch_bounds__(kBlockThreads) void k_copy_mix(CopyMixParams p, int64_t tile0) {
    __shared__ uint4 s_in[kTile * kMaxPieces];
    const int tid = threadIdx.x;
    const int64_t r0 = (tile0 + blockIdx.x) * kTile;
    if (r0 >= p.rows) return;                   // workgroup-uniform
    const int nrows = (int)min((int64_t)kTile, p.rows - r0);
    const int in_n = nrows * p.rp, out_n = nrows * p.wp;
    const uint8_t* src = p.src + r0 * p.rp * 16;
    uint8_t* dst = p.dst + r0 * p.wp * 16;
    uint4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; k++) {
        const int j = tid + kBlockThreads * k;
        if (j < in_n) v[k] = ld_stream16(src + 16 * j);
    }
#pragma unroll
    for (int k = 0; k < kLoads; k++) {
        const int j = tid + kBlockThreads * k;
        if (j < in_n) s_in[j] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kLoads; k++) {
        const int q = tid + kBlockThreads * k;
        if (q >= out_n) break;
        const int row = q / p.wp, c = q - row * p.wp;
        const uint4* in = s_in + row * p.rp;
        uint4 o = in[c % p.rp];
        for (int i = c + p.wp; i < p.rp; i += p.wp) {
            o.x ^= in[i].x;
            o.y ^= in[i].y;
            o.z ^= in[i].z;
            o.w ^= in[i].w;
        }
        st_stream16(dst + 16 * q, o);
    }
}

}  // namespace

extern "C" int gcache_bench_copy_mix(const void* src, void* dst, int64_t rows, int32_t read_bytes,
                                     int32_t write_bytes, hipStream_t stream) {
    if (rows < 0 || read_bytes < 16 || write_bytes < 16 || read_bytes > 16 * kMaxPieces ||
        write_bytes > 16 * kMaxPieces || read_bytes % 16 || write_bytes % 16)
        return -2;
    if (rows == 0) return 0;
    if (!src || !dst) return -1;
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return -3;
    CopyMixParams p{static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows, read_bytes / 16,
                    write_bytes / 16};
    const int64_t tiles = (rows + kTile - 1) / kTile;
    constexpr int64_t kMaxGrid = int64_t(1) << 30;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxGrid) {
        const int64_t n = tiles - t0 < kMaxGrid ? tiles - t0 : kMaxGrid;
        void* args[] = {&p, const_cast<int64_t*>(&t0)};
        if (hipLaunchKernel(reinterpret_cast<const void*>(k_copy_mix), dim3((unsigned)n), dim3(kBlockThreads), args,
                            0, stream) != hipSuccess)
            return -6;
    }
    return 0;
}
