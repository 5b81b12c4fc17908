// bench_ceiling.hip -- libgcache_bench.so: the same-mix copy that bench.py
// uses as an on-device ceiling for the cache operations (declared in
// include/gcache_bench.h).  Not part of the cache path.
#include <hip/hip_ext.h>

#include "../../include/gcache_bench.h"
#include "gcache_device.h"

namespace {

using namespace gcache;

constexpr int kMaxPieces = 72;                  // 1152 bytes per row at most
constexpr int kMaxStaged = 16 * kMaxPieces;     // input pieces staged per workgroup at most (18 KiB)
constexpr int kMaxLoads = 18;                   // input pieces per thread at most

struct CopyMixParams {
    const uint8_t* src;
    uint8_t* dst;
    int64_t rows;
    int32_t rp, wp;                             // 16-byte pieces read / written per row
    int32_t group;                              // rows per workgroup
};

// One workgroup per `group` rows: every input piece of the group is loaded
// (all loads in flight), staged in LDS, then the output pieces are stored,
// the way the cache kernels stage their tiles.
__global__ __launch_bounds__(1024) void k_copy_mix(CopyMixParams p, int64_t g0) {
    extern __shared__ uint4 s_in[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t r0 = (g0 + blockIdx.x) * p.group;
    if (r0 >= p.rows) return;                   // workgroup-uniform
    const int nrows = (int)min((int64_t)p.group, p.rows - r0);
    const int in_n = nrows * p.rp, out_n = nrows * p.wp;
    const uint8_t* src = p.src + r0 * p.rp * 16;
    uint8_t* dst = p.dst + r0 * p.wp * 16;
    uint4 v[kMaxLoads];
#pragma unroll
    for (int k = 0; k < kMaxLoads; k++) {
        const int j = tid + nt * k;
        if (j < in_n) v[k] = ld_stream16(src + 16 * j);
    }
#pragma unroll
    for (int k = 0; k < kMaxLoads; k++) {
        const int j = tid + nt * k;
        if (j < in_n) s_in[j] = v[k];
    }
    __syncthreads();
    for (int q = tid; q < out_n; q += nt) {
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

// No wave touches memory: the store is behind a condition no workgroup
// meets (blockIdx.x never reaches 2^31), so the kernel is not empty code.
__global__ __launch_bounds__(1024) void k_empty(int* never) {
    if (blockIdx.x == 0x80000000u && threadIdx.x == 0) *never = 0;
}

}  // namespace

extern "C" int gcache_bench_copy_mix(const void* src, void* dst, int64_t rows, int32_t read_bytes,
                                     int32_t write_bytes, int32_t rows_per_group, int32_t threads,
                                     hipStream_t stream) {
    if (rows < 0 || read_bytes < 16 || write_bytes < 16 || read_bytes > 16 * kMaxPieces ||
        write_bytes > 16 * kMaxPieces || read_bytes % 16 || write_bytes % 16)
        return -2;
    if (threads < 64 || threads > 1024 || threads % 64 || rows_per_group < 1)
        return -2;
    const int64_t staged = (int64_t)rows_per_group * (read_bytes / 16);
    if (staged > kMaxStaged) return -2;             // (then at most kMaxLoads pieces per lane)
    if (rows == 0) return 0;
    if (!src || !dst) return -1;
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return -3;
    CopyMixParams p{static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows, read_bytes / 16,
                    write_bytes / 16, rows_per_group};
    const int64_t groups = (rows + rows_per_group - 1) / rows_per_group;
    constexpr int64_t kMaxGrid = int64_t(1) << 30;
    for (int64_t g0 = 0; g0 < groups; g0 += kMaxGrid) {
        const int64_t n = groups - g0 < kMaxGrid ? groups - g0 : kMaxGrid;
        void* args[] = {&p, const_cast<int64_t*>(&g0)};
        if (hipLaunchKernel(reinterpret_cast<const void*>(k_copy_mix), dim3((unsigned)n), dim3(threads), args,
                            (size_t)staged * 16, stream) != hipSuccess)
            return -6;
    }
    return 0;
}

extern "C" int gcache_bench_empty_grid(int64_t groups, int32_t threads, hipEvent_t start, hipEvent_t stop,
                                       hipStream_t stream) {
    if (groups < 1 || groups >= (int64_t(1) << 31) || threads < 64 || threads > 1024 || threads % 64)
        return -2;
    int* never = nullptr;
    void* args[] = {&never};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(k_empty), dim3((unsigned)groups), dim3(threads), args,
                              0, stream, start, stop, 0) == hipSuccess ? 0 : -6;
}
