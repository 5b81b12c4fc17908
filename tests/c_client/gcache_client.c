/*
 * gcache_client.c -- a plain C99 program that uses libgcache.so only through
 * include/gcache.h, the way an application embedding the library would:
 * buffers from hipMalloc, a stream of its own, status codes checked after
 * every call.  No Python and no torch are involved.
 *
 *   gcache_client host
 *       Calls the host-only entry points and a few rejected calls (fake
 *       device addresses that the library never dereferences, because the
 *       arguments fail validation first).  Prints key=value lines.
 *
 *   gcache_client roundtrip FMT DIR T NB BS B MAXB TOTAL
 *       FMT is nvfp4 or fp8.  Reads DIR/kv_c.bin (uint16 [T,512]),
 *       DIR/k_pe.bin (uint16 [T,64]), DIR/slots.bin (int64 [T]),
 *       DIR/block_table.bin (int32 [B,MAXB]), DIR/ws.bin and DIR/ss.bin
 *       (int32 [B]).  Fills a cache of NB blocks x BS entries with 0xA5,
 *       writes the tokens into it, gathers TOTAL rows back, and writes
 *       DIR/cache.bin and DIR/out.bin (uint16 [TOTAL,576]).  The gather's
 *       own duration is taken with two events bound to that kernel
 *       (gcache_time_next_launch) and printed as gather_kernel_ms=...
 *
 * Exit status: 0 on success, 1 on a usage or I/O error, 2 when a library or
 * HIP call fails (its status is printed first).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gcache.h"

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));          \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

#define GC_OK(call)                                                                    \
    do {                                                                               \
        int s_ = (call);                                                               \
        if (s_ != GCACHE_OK) {                                                         \
            fprintf(stderr, "%s returned %d (%s)\n", #call, s_, gcache_status_string(s_)); \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

static void print_layout(const char* name, const gcache_nvfp4_kv_layout* L) {
    printf("%s=%lld,%lld,%lld,%lld,%lld,%lld,%lld,%lld\n", name, (long long)L->data_offset,
           (long long)L->data_token_stride, (long long)L->data_head_stride, (long long)L->scale_offset,
           (long long)L->scale_token_stride, (long long)L->scale_head_stride, (long long)L->side_stride,
           (long long)L->block_stride);
}

static int host_mode(void) {
    gcache_nvfp4_kv_layout L;
    printf("entry_bytes_nvfp4=%lld\n", (long long)gcache_entry_bytes(GCACHE_NVFP4_DS_MLA));
    printf("entry_bytes_fp8=%lld\n", (long long)gcache_entry_bytes(GCACHE_FP8_DS_MLA));
    printf("full_dim_128=%d\n", gcache_nvfp4_full_dim(128));
    printf("full_dim_24=%d\n", gcache_nvfp4_full_dim(24));
    GC_OK(gcache_nvfp4_kv_split_layout(16, 8, 128, &L));
    print_layout("split_nhd_16_8_128", &L);
    GC_OK(gcache_nvfp4_kv_split_layout_hnd(16, 8, 128, &L));
    print_layout("split_hnd_16_8_128", &L);
    printf("split_bad_head=%d\n", gcache_nvfp4_kv_split_layout(16, 8, 100, &L));

    /* chunked context: 3 requests, 1000-row workspace, blocks of 64 */
    {
        const int32_t lens[3] = {700, 0, 1500};
        int32_t chunk_rows = 0, num_chunks = 0, c;
        GC_OK(gcache_context_chunk_plan(lens, 3, 1000, 64, &chunk_rows, &num_chunks));
        printf("chunk_plan=%d,%d\n", chunk_rows, num_chunks);
        for (c = 0; c < num_chunks; c++) {
            int32_t ss[3], ws[3];
            int64_t total = -1;
            GC_OK(gcache_context_chunk(lens, 3, chunk_rows, c, ss, ws, &total));
            printf("chunk_%d=%d,%d,%d|%d,%d,%d|%lld\n", c, ss[0], ss[1], ss[2], ws[0], ws[1], ws[2],
                   (long long)total);
        }
        {
            int32_t ss[3], ws[3];
            int64_t total = -1;
            printf("chunk_out_of_range=%d\n", gcache_context_chunk(lens, 3, chunk_rows, num_chunks, ss, ws, &total));
            printf("chunk_null_output=%d\n", gcache_context_chunk(lens, 3, chunk_rows, 0, NULL, ws, &total));
        }
    }

    /* rejected before any device work: fake, never dereferenced addresses */
    {
        void* a = (void*)(uintptr_t)0x10000;
        printf("write_null_input=%d\n",
               gcache_cache_write_nvfp4_ds_mla(NULL, a, a, (const int64_t*)a, 4, 512, 64, 2, 64, 64 * 352, 352,
                                               NULL));
        printf("write_short_entry=%d\n",
               gcache_cache_write_nvfp4_ds_mla(a, a, a, (const int64_t*)a, 4, 512, 64, 2, 64, 64 * 352, 336,
                                               NULL));
        printf("write_misaligned=%d\n",
               gcache_cache_write_nvfp4_ds_mla((char*)a + 8, a, a, (const int64_t*)a, 4, 512, 64, 2, 64,
                                               64 * 352, 352, NULL));
        printf("gather_no_requests=%d\n",
               gcache_cache_gather_upconvert_fp8_ds_mla(a, a, 10, 576, (const int32_t*)a, 8, (const int32_t*)a,
                                                        (const int32_t*)a, 0, 4, 64, 64 * 656, 656, NULL));
        printf("gather_empty=%d\n",
               gcache_cache_gather_upconvert_nvfp4_ds_mla(NULL, NULL, 0, 576, NULL, 8, NULL, NULL, 0, 4, 64,
                                                          64 * 352, 352, NULL));
    }
    printf("status_unsupported=%s\n", gcache_status_string(GCACHE_ERR_UNSUPPORTED));
    return 0;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    FILE* f;
    void* buf = malloc(bytes ? bytes : 1);
    snprintf(path, sizeof path, "%s/%s", dir, name);
    f = fopen(path, "rb");
    if (!f || !buf || fread(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
        exit(1);
    }
    fclose(f);
    return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
    char path[4096];
    FILE* f;
    snprintf(path, sizeof path, "%s/%s", dir, name);
    f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(1);
    }
    fclose(f);
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static int roundtrip_mode(int argc, char** argv) {
    const char *fmt, *dir;
    long long T, NB, BS, B, MAXB, TOTAL;
    int nvfp4;
    int64_t eb;
    size_t cache_bytes, out_bytes;
    void *h_kv, *h_pe, *h_sl, *h_bt, *h_ws, *h_ss, *h_cache, *h_out;
    void *kv, *pe, *sl, *bt, *ws, *ss, *cache, *out;
    hipStream_t stream;
    hipEvent_t ev_start, ev_stop;
    float gather_ms = 0.0f;

    if (argc != 10) {
        fprintf(stderr, "usage: gcache_client roundtrip FMT DIR T NB BS B MAXB TOTAL\n");
        return 1;
    }
    fmt = argv[2];
    dir = argv[3];
    T = atoll(argv[4]);
    NB = atoll(argv[5]);
    BS = atoll(argv[6]);
    B = atoll(argv[7]);
    MAXB = atoll(argv[8]);
    TOTAL = atoll(argv[9]);
    nvfp4 = strcmp(fmt, "nvfp4") == 0;
    if (!nvfp4 && strcmp(fmt, "fp8") != 0) {
        fprintf(stderr, "FMT must be nvfp4 or fp8\n");
        return 1;
    }
    if (T < 0 || NB <= 0 || BS <= 0 || B <= 0 || MAXB <= 0 || TOTAL < 0) {
        fprintf(stderr, "sizes out of range\n");
        return 1;
    }
    eb = gcache_entry_bytes(nvfp4 ? GCACHE_NVFP4_DS_MLA : GCACHE_FP8_DS_MLA);
    cache_bytes = (size_t)NB * (size_t)BS * (size_t)eb;
    out_bytes = (size_t)TOTAL * 576 * 2;

    h_kv = read_file(dir, "kv_c.bin", (size_t)T * 512 * 2);
    h_pe = read_file(dir, "k_pe.bin", (size_t)T * 64 * 2);
    h_sl = read_file(dir, "slots.bin", (size_t)T * 8);
    h_bt = read_file(dir, "block_table.bin", (size_t)B * (size_t)MAXB * 4);
    h_ws = read_file(dir, "ws.bin", (size_t)B * 4);
    h_ss = read_file(dir, "ss.bin", (size_t)B * 4);

    HIP_OK(hipStreamCreate(&stream));
    kv = to_device(h_kv, (size_t)T * 512 * 2);
    pe = to_device(h_pe, (size_t)T * 64 * 2);
    sl = to_device(h_sl, (size_t)T * 8);
    bt = to_device(h_bt, (size_t)B * (size_t)MAXB * 4);
    ws = to_device(h_ws, (size_t)B * 4);
    ss = to_device(h_ss, (size_t)B * 4);
    HIP_OK(hipMalloc(&cache, cache_bytes));
    HIP_OK(hipMalloc(&out, out_bytes ? out_bytes : 16));
    HIP_OK(hipMemsetAsync(cache, 0xA5, cache_bytes, stream));
    if (out_bytes) HIP_OK(hipMemsetAsync(out, 0x00, out_bytes, stream));
    HIP_OK(hipEventCreate(&ev_start));
    HIP_OK(hipEventCreate(&ev_stop));

    if (nvfp4) {
        GC_OK(gcache_cache_write_nvfp4_ds_mla(kv, pe, cache, (const int64_t*)sl, T, 512, 64, NB, (int32_t)BS,
                                              BS * eb, eb, stream));
        GC_OK(gcache_time_next_launch(ev_start, ev_stop));
        GC_OK(gcache_cache_gather_upconvert_nvfp4_ds_mla(cache, out, TOTAL, 576, (const int32_t*)bt, MAXB,
                                                         (const int32_t*)ws, (const int32_t*)ss, (int32_t)B, NB,
                                                         (int32_t)BS, BS * eb, eb, stream));
    } else {
        GC_OK(gcache_cache_write_fp8_ds_mla(kv, pe, cache, (const int64_t*)sl, T, 512, 64, NB, (int32_t)BS,
                                            BS * eb, eb, stream));
        GC_OK(gcache_time_next_launch(ev_start, ev_stop));
        GC_OK(gcache_cache_gather_upconvert_fp8_ds_mla(cache, out, TOTAL, 576, (const int32_t*)bt, MAXB,
                                                       (const int32_t*)ws, (const int32_t*)ss, (int32_t)B, NB,
                                                       (int32_t)BS, BS * eb, eb, stream));
    }
    HIP_OK(hipStreamSynchronize(stream));
    if (TOTAL > 0) {                     /* the gather launched and consumed the hook */
        HIP_OK(hipEventElapsedTime(&gather_ms, ev_start, ev_stop));
        printf("gather_kernel_ms=%.6f\n", gather_ms);
    } else {
        GC_OK(gcache_time_next_launch(NULL, NULL));   /* nothing launched: disarm */
    }
    HIP_OK(hipEventDestroy(ev_start));
    HIP_OK(hipEventDestroy(ev_stop));

    h_cache = malloc(cache_bytes);
    h_out = malloc(out_bytes ? out_bytes : 1);
    if (!h_cache || !h_out) {
        fprintf(stderr, "out of host memory\n");
        return 1;
    }
    HIP_OK(hipMemcpy(h_cache, cache, cache_bytes, hipMemcpyDeviceToHost));
    if (out_bytes) HIP_OK(hipMemcpy(h_out, out, out_bytes, hipMemcpyDeviceToHost));
    write_file(dir, "cache.bin", h_cache, cache_bytes);
    write_file(dir, "out.bin", h_out, out_bytes);

    HIP_OK(hipFree(kv));
    HIP_OK(hipFree(pe));
    HIP_OK(hipFree(sl));
    HIP_OK(hipFree(bt));
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(ss));
    HIP_OK(hipFree(cache));
    HIP_OK(hipFree(out));
    HIP_OK(hipStreamDestroy(stream));
    free(h_kv);
    free(h_pe);
    free(h_sl);
    free(h_bt);
    free(h_ws);
    free(h_ss);
    free(h_cache);
    free(h_out);
    printf("roundtrip %s ok: %lld tokens written, %lld rows gathered\n", fmt, T, TOTAL);
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode();
    if (argc >= 2 && strcmp(argv[1], "roundtrip") == 0) return roundtrip_mode(argc, argv);
    fprintf(stderr, "usage: gcache_client host | roundtrip FMT DIR T NB BS B MAXB TOTAL\n");
    return 1;
}
