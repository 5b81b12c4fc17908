/*
 * gcache_bench.h -- C ABI of libgcache_bench.so, a measurement helper that
 * ships beside libgcache.so.  It is not part of the cache path: bench.py
 * uses it to measure, on the same device, the bandwidth a plain stream
 * with the same byte pattern as one of the cache operations reaches, so
 * each operation can be reported as a fraction of that same-mix ceiling as
 * well as of the HBM peak.
 */
#ifndef GCACHE_BENCH_H
#define GCACHE_BENCH_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Same-mix row copy: for every row r < rows, reads read_bytes contiguous
 * bytes at src + r * read_bytes and writes write_bytes contiguous bytes at
 * dst + r * write_bytes, built from the row's input 16-byte pieces (piece c
 * of the output is input piece c % (read_bytes / 16) when the output is
 * wider, the XOR of input pieces c, c + w, c + 2w, ... (w = write_bytes / 16)
 * when it is narrower), so every input byte is used.  Workgroups of
 * `threads` lanes take rows_per_group rows each and stage them through LDS
 * like the cache kernels, with no block-table walk and no format
 * conversion; bench.py times several workgroup shapes and keeps the
 * fastest as the ceiling.
 *  src, dst  device pointers, 16-byte aligned, owned by the caller
 *  read_bytes, write_bytes  multiples of 16 in [16, 1152]
 *  rows_per_group >= 1 with rows_per_group * read_bytes <= 18432,
 *  threads a multiple of 64 in [64, 1024]
 * Returns 0, -1 for a null pointer, -2 for sizes or shapes out of range,
 * -3 for a misaligned pointer, -6 when the launch fails.  Enqueued on
 * `stream`; nothing is allocated or synchronized.
 */
int gcache_bench_copy_mix(const void* src, void* dst, int64_t rows, int32_t read_bytes,
                          int32_t write_bytes, int32_t rows_per_group, int32_t threads,
                          hipStream_t stream);

/*
 * Launch cost floor: one launch of `groups` workgroups of `threads` lanes
 * whose waves exit without touching memory, with `start` / `stop` (HIP
 * events created by the caller, or NULL) bound to the kernel's own begin and
 * end as for the cache entry points' timing hook, so the elapsed time between
 * them is what any kernel of that grid pays before and after its work.
 *  groups in [1, 2^31), threads a multiple of 64 in [64, 1024]
 * Returns 0, -2 for a grid out of range, -6 when the launch fails.  Enqueued
 * on `stream`; nothing is allocated or synchronized.
 */
int gcache_bench_empty_grid(int64_t groups, int32_t threads, hipEvent_t start, hipEvent_t stop,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GCACHE_BENCH_H */
