// gcache_abi.hip -- the extern "C" entry points declared in include/gcache.h.
//
// Each entry point checks its arguments on the host (returning a negative
// gcache_status and launching nothing when one is rejected, in the spirit of
// the length assertion that guards a kernel grid in the vLLM PR #48642
// digest, "Implementation breakdown" item 1), checks once per device that
// the current device is a gfx950, and enqueues one kernel on the caller's
// stream.  Nothing here allocates, frees or synchronizes.
#include <atomic>
#include <cstring>

#include "../../include/gcache.h"
#include "gcache_internal.h"

using namespace gcache;

// Timing events armed by gcache_time_next_launch, per host thread.
LaunchTiming& gcache::launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GCACHE_ERR_DEVICE;
    if (dev >= kMaxDevices) return GCACHE_ERR_UNSUPPORTED;
    int state = g_arch_state[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GCACHE_ERR_DEVICE;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_arch_state[dev].store(state, std::memory_order_relaxed);
    }
    return state > 0 ? GCACHE_OK : GCACHE_ERR_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b without signed overflow (both non-negative); false when it overflows.
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

BlockDiv make_div(int32_t block_size) {
    BlockDiv d{block_size, -1};
    if ((block_size & (block_size - 1)) == 0) d.shift = __builtin_ctz((unsigned)block_size);
    return d;
}

int log2_or_minus1(int v) { return (v > 0 && (v & (v - 1)) == 0) ? __builtin_ctz((unsigned)v) : -1; }

int launched(hipError_t e) { return e == hipSuccess ? GCACHE_OK : GCACHE_ERR_LAUNCH; }

// Shared checks of the DS-MLA cache geometry.
int check_ds_cache(const void* cache, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                   int64_t entry_stride, int64_t entry_bytes) {
    if (num_blocks < 0 || block_size <= 0 || entry_stride < entry_bytes) return GCACHE_ERR_SHAPE;
    int64_t need;
    if (!mul_ok(block_size, entry_stride, &need) || block_stride < need) return GCACHE_ERR_SHAPE;
    if (!mul_ok(num_blocks, block_stride, &need)) return GCACHE_ERR_SHAPE;
    if (!aligned(cache, 16) || block_stride % 16 || entry_stride % 16) return GCACHE_ERR_ALIGN;
    return GCACHE_OK;
}

int ds_write(bool nvfp4, const void* kv_c, const void* k_pe, void* kv_cache,
             const int64_t* slot_mapping, int64_t num_tokens, int64_t kv_c_stride,
             int64_t k_pe_stride, int64_t num_blocks, int32_t block_size, int64_t block_stride,
             int64_t entry_stride, hipStream_t stream) {
    if (num_tokens < 0) return GCACHE_ERR_SHAPE;
    if (num_tokens == 0) return GCACHE_OK;
    if (!kv_c || !k_pe || !kv_cache || !slot_mapping) return GCACHE_ERR_NULL;
    if (kv_c_stride < kNope || k_pe_stride < kRope) return GCACHE_ERR_SHAPE;
    int rc = check_ds_cache(kv_cache, num_blocks, block_size, block_stride, entry_stride,
                            nvfp4 ? kNvEntry : kF8Entry);
    if (rc) return rc;
    if (!aligned(kv_c, 16) || !aligned(k_pe, 16) || kv_c_stride % 8 || k_pe_stride % 8)
        return GCACHE_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    DsMlaWriteParams p;
    p.kv_c = static_cast<const uint16_t*>(kv_c);
    p.k_pe = static_cast<const uint16_t*>(k_pe);
    p.cache = static_cast<uint8_t*>(kv_cache);
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.kv_c_stride = kv_c_stride;
    p.k_pe_stride = k_pe_stride;
    p.block_stride = block_stride;
    p.entry_stride = entry_stride;
    p.div = make_div(block_size);
    return launched(nvfp4 ? launch_write_nvfp4_ds_mla(p, stream) : launch_write_fp8_ds_mla(p, stream));
}

// Shared checks of the gather walk arguments.
int check_walk(int64_t total_tokens, const int32_t* block_table, int64_t block_table_stride,
               const int32_t* workspace_starts, int32_t batch_size) {
    if (!block_table || !workspace_starts) return GCACHE_ERR_NULL;
    if (batch_size <= 0 || block_table_stride <= 0 || total_tokens > INT32_MAX)
        return GCACHE_ERR_SHAPE;
    return GCACHE_OK;
}

enum { kFmtNvfp4, kFmtFp8, kFmtBf16 };

int ds_gather(int fmt, const void* src_cache, void* dst, int64_t total_tokens,
              int64_t dst_stride, const int32_t* block_table, int64_t block_table_stride,
              const int32_t* workspace_starts, const int32_t* seq_starts, int32_t batch_size,
              int64_t num_blocks, int32_t block_size, int64_t block_stride, int64_t entry_stride,
              hipStream_t stream) {
    if (total_tokens < 0) return GCACHE_ERR_SHAPE;
    if (total_tokens == 0) return GCACHE_OK;
    if (!src_cache || !dst) return GCACHE_ERR_NULL;
    int rc = check_walk(total_tokens, block_table, block_table_stride, workspace_starts, batch_size);
    if (rc) return rc;
    if (dst_stride < kRow) return GCACHE_ERR_SHAPE;
    if ((rc = check_ds_cache(src_cache, num_blocks, block_size, block_stride, entry_stride,
                             fmt == kFmtNvfp4 ? kNvEntry : fmt == kFmtFp8 ? kF8Entry : 2 * kRow)))
        return rc;
    if (!aligned(dst, 16) || dst_stride % 8) return GCACHE_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    DsMlaGatherParams p;
    p.cache = static_cast<const uint8_t*>(src_cache);
    p.dst = static_cast<uint16_t*>(dst);
    p.total = total_tokens;
    p.dst_stride = dst_stride;
    p.block_table = block_table;
    p.bt_stride = block_table_stride;
    p.ws = workspace_starts;
    p.seq_starts = seq_starts;
    p.batch = batch_size;
    p.num_blocks = num_blocks;
    p.block_stride = block_stride;
    p.entry_stride = entry_stride;
    p.div = make_div(block_size);
    return launched(fmt == kFmtNvfp4 ? launch_gather_nvfp4_ds_mla(p, stream)
                    : fmt == kFmtFp8 ? launch_gather_fp8_ds_mla(p, stream)
                                     : launch_gather_bf16(p, stream));
}

int check_kv(int32_t num_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
             const gcache_nvfp4_kv_layout* L, const float* k_scale, const float* v_scale,
             const void* cache) {
    if (!L || !k_scale || !v_scale || !cache) return GCACHE_ERR_NULL;
    if (num_heads <= 0 || head_size <= 0 || head_size % 16 || head_size > 1024 ||
        num_blocks < 0 || block_size <= 0)
        return GCACHE_ERR_SHAPE;
    const int64_t v[8] = {L->data_offset, L->data_token_stride, L->data_head_stride,
                          L->scale_offset, L->scale_token_stride, L->scale_head_stride,
                          L->side_stride, L->block_stride};
    for (int64_t x : v)
        if (x < 0) return GCACHE_ERR_SHAPE;
    int64_t tmp;
    if (!mul_ok(num_blocks, L->block_stride, &tmp) || !mul_ok(num_blocks, block_size, &tmp))
        return GCACHE_ERR_SHAPE;
    // data rows are read and written 8 (write) or 4 (gather) bytes at a time
    if (!aligned(cache, 16) || L->data_offset % 8 || L->data_token_stride % 8 ||
        L->data_head_stride % 8 || L->side_stride % 8 || L->block_stride % 8)
        return GCACHE_ERR_ALIGN;
    return GCACHE_OK;
}

KvLayout to_layout(const gcache_nvfp4_kv_layout* L) {
    KvLayout k;
    k.data_offset = L->data_offset;
    k.data_token_stride = L->data_token_stride;
    k.data_head_stride = L->data_head_stride;
    k.scale_offset = L->scale_offset;
    k.scale_token_stride = L->scale_token_stride;
    k.scale_head_stride = L->scale_head_stride;
    k.side_stride = L->side_stride;
    k.block_stride = L->block_stride;
    return k;
}

bool kv_strides_ok(const void* base, int64_t token_stride, int64_t head_stride) {
    return aligned(base, 16) && token_stride >= 0 && head_stride >= 0 && token_stride % 8 == 0 &&
           head_stride % 8 == 0;
}

}  // namespace

extern "C" {

int64_t gcache_entry_bytes(gcache_format format) {
    switch (format) {
        case GCACHE_NVFP4_DS_MLA: return kNvEntry;
        case GCACHE_FP8_DS_MLA: return kF8Entry;
    }
    return -1;
}

int32_t gcache_nvfp4_full_dim(int32_t head_size) {
    if (head_size <= 0 || head_size % 16) return -1;
    return head_size / 2 + head_size / 16;
}

int gcache_time_next_launch(hipEvent_t start, hipEvent_t stop) {
    launch_timing() = LaunchTiming{start, stop};
    return GCACHE_OK;
}

const char* gcache_status_string(int status) {
    switch (status) {
        case GCACHE_OK: return "ok";
        case GCACHE_ERR_NULL: return "null pointer argument";
        case GCACHE_ERR_SHAPE: return "size or stride out of range";
        case GCACHE_ERR_ALIGN: return "misaligned base pointer or stride";
        case GCACHE_ERR_UNSUPPORTED: return "unsupported device or shape (gfx950 required)";
        case GCACHE_ERR_DEVICE: return "HIP device query failed";
        case GCACHE_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int gcache_cache_write_nvfp4_ds_mla(const void* kv_c, const void* k_pe, void* kv_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens,
                                    int64_t kv_c_stride, int64_t k_pe_stride, int64_t num_blocks,
                                    int32_t block_size, int64_t block_stride, int64_t entry_stride,
                                    hipStream_t stream) {
    return ds_write(true, kv_c, k_pe, kv_cache, slot_mapping, num_tokens, kv_c_stride, k_pe_stride,
                    num_blocks, block_size, block_stride, entry_stride, stream);
}

int gcache_cache_write_fp8_ds_mla(const void* kv_c, const void* k_pe, void* kv_cache,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  int64_t kv_c_stride, int64_t k_pe_stride, int64_t num_blocks,
                                  int32_t block_size, int64_t block_stride, int64_t entry_stride,
                                  hipStream_t stream) {
    return ds_write(false, kv_c, k_pe, kv_cache, slot_mapping, num_tokens, kv_c_stride, k_pe_stride,
                    num_blocks, block_size, block_stride, entry_stride, stream);
}

int gcache_cache_gather_upconvert_nvfp4_ds_mla(const void* src_cache, void* dst,
                                               int64_t total_tokens, int64_t dst_stride,
                                               const int32_t* block_table,
                                               int64_t block_table_stride,
                                               const int32_t* workspace_starts,
                                               const int32_t* seq_starts, int32_t batch_size,
                                               int64_t num_blocks, int32_t block_size,
                                               int64_t block_stride, int64_t entry_stride,
                                               hipStream_t stream) {
    return ds_gather(kFmtNvfp4, src_cache, dst, total_tokens, dst_stride, block_table, block_table_stride,
                     workspace_starts, seq_starts, batch_size, num_blocks, block_size, block_stride,
                     entry_stride, stream);
}

int gcache_cache_gather_upconvert_fp8_ds_mla(const void* src_cache, void* dst,
                                             int64_t total_tokens, int64_t dst_stride,
                                             const int32_t* block_table,
                                             int64_t block_table_stride,
                                             const int32_t* workspace_starts,
                                             const int32_t* seq_starts, int32_t batch_size,
                                             int64_t num_blocks, int32_t block_size,
                                             int64_t block_stride, int64_t entry_stride,
                                             hipStream_t stream) {
    return ds_gather(kFmtFp8, src_cache, dst, total_tokens, dst_stride, block_table, block_table_stride,
                     workspace_starts, seq_starts, batch_size, num_blocks, block_size, block_stride,
                     entry_stride, stream);
}

int gcache_convert_req_index_to_global_index(const int32_t* req_id, int64_t num_req_id,
                                             const int32_t* token_indices, int64_t num_tokens,
                                             int32_t topk, int64_t token_indices_stride,
                                             const int32_t* block_table, int32_t batch_size,
                                             int64_t block_table_stride, int32_t block_size,
                                             int64_t num_blocks, int32_t* out, int64_t out_stride,
                                             hipStream_t stream) {
    // the length check of the pages: one request id per token row, exactly
    if (num_req_id != num_tokens || num_tokens < 0 || topk < 0) return GCACHE_ERR_SHAPE;
    if (num_tokens == 0 || topk == 0) return GCACHE_OK;
    if (!req_id || !token_indices || !block_table || !out) return GCACHE_ERR_NULL;
    if (token_indices_stride < topk || out_stride < topk || batch_size <= 0 ||
        block_table_stride <= 0 || block_size <= 0 || num_blocks < 0)
        return GCACHE_ERR_SHAPE;
    int64_t slots;
    if (!mul_ok(num_blocks, block_size, &slots) || slots > INT32_MAX) return GCACHE_ERR_SHAPE;
    if (!aligned(req_id, 4) || !aligned(token_indices, 4) || !aligned(block_table, 4) || !aligned(out, 4))
        return GCACHE_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    SparseIndexParams p;
    p.req_id = req_id;
    p.token_indices = token_indices;
    p.out = out;
    p.num_tokens = num_tokens;
    p.ti_stride = token_indices_stride;
    p.out_stride = out_stride;
    p.topk = topk;
    p.waves_per_row = 0;                                 // set by the launcher
    p.vec16 = topk % 4 == 0 && token_indices_stride % 4 == 0 && out_stride % 4 == 0 &&
              aligned(token_indices, 16) && aligned(out, 16);
    p.block_table = block_table;
    p.bt_stride = block_table_stride;
    p.batch = batch_size;
    p.num_blocks = num_blocks;
    p.div = make_div(block_size);
    return launched(launch_convert_req_index(p, stream));
}

int gcache_context_chunk_plan(const int32_t* context_lens, int32_t batch_size,
                              int64_t workspace_rows, int32_t block_size,
                              int32_t* chunk_rows, int32_t* num_chunks) {
    if (!context_lens || !chunk_rows || !num_chunks) return GCACHE_ERR_NULL;
    if (batch_size <= 0 || block_size <= 0 || workspace_rows < 0) return GCACHE_ERR_SHAPE;
    int32_t longest = 0;
    for (int32_t b = 0; b < batch_size; b++) {
        if (context_lens[b] < 0) return GCACHE_ERR_SHAPE;
        longest = context_lens[b] > longest ? context_lens[b] : longest;
    }
    // a chunk's rows are addressed with int32 workspace_starts
    const int64_t usable = workspace_rows < INT32_MAX ? workspace_rows : INT32_MAX;
    const int64_t c = usable / batch_size / block_size * block_size;
    if (c <= 0) return GCACHE_ERR_SHAPE;                    // not one block per request
    *chunk_rows = (int32_t)c;
    *num_chunks = (int32_t)((longest + c - 1) / c);
    return GCACHE_OK;
}

int gcache_context_chunk(const int32_t* context_lens, int32_t batch_size, int32_t chunk_rows,
                         int32_t chunk, int32_t* seq_starts, int32_t* workspace_starts,
                         int64_t* total_rows) {
    if (!context_lens || !seq_starts || !workspace_starts || !total_rows) return GCACHE_ERR_NULL;
    if (batch_size <= 0 || chunk_rows <= 0 || chunk < 0) return GCACHE_ERR_SHAPE;
    const int64_t start = (int64_t)chunk * chunk_rows;
    int64_t total = 0;
    bool any = false;
    for (int32_t b = 0; b < batch_size; b++) {
        if (context_lens[b] < 0) return GCACHE_ERR_SHAPE;
        any = any || context_lens[b] > start;
    }
    if (!any || start > INT32_MAX) return GCACHE_ERR_SHAPE;  // chunk past the longest context
    for (int32_t b = 0; b < batch_size; b++) {
        int64_t len = context_lens[b] - start;
        len = len < 0 ? 0 : (len > chunk_rows ? chunk_rows : len);
        if (total > INT32_MAX) return GCACHE_ERR_SHAPE;
        seq_starts[b] = (int32_t)start;
        workspace_starts[b] = (int32_t)total;
        total += len;
    }
    *total_rows = total;
    return GCACHE_OK;
}

int gcache_cache_gather_bf16(const void* src_cache, void* dst, int64_t total_tokens,
                             int64_t dst_stride, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* workspace_starts,
                             const int32_t* seq_starts, int32_t batch_size, int64_t num_blocks,
                             int32_t block_size, int64_t block_stride, int64_t entry_stride,
                             hipStream_t stream) {
    return ds_gather(kFmtBf16, src_cache, dst, total_tokens, dst_stride, block_table, block_table_stride,
                     workspace_starts, seq_starts, batch_size, num_blocks, block_size, block_stride,
                     entry_stride, stream);
}

int gcache_nvfp4_kv_split_layout(int32_t block_size, int32_t num_heads, int32_t head_size,
                                 gcache_nvfp4_kv_layout* out) {
    if (!out) return GCACHE_ERR_NULL;
    if (block_size <= 0 || num_heads <= 0 || head_size <= 0 || head_size % 16)
        return GCACHE_ERR_SHAPE;
    const int64_t data_row = head_size / 2, scale_row = head_size / 16;
    const int64_t side = (int64_t)block_size * num_heads * (data_row + scale_row);
    out->data_offset = 0;
    out->data_token_stride = (int64_t)num_heads * data_row;
    out->data_head_stride = data_row;
    out->scale_offset = (int64_t)block_size * num_heads * data_row;
    out->scale_token_stride = (int64_t)num_heads * scale_row;
    out->scale_head_stride = scale_row;
    out->side_stride = side;
    out->block_stride = 2 * side;
    return GCACHE_OK;
}

int gcache_nvfp4_kv_split_layout_hnd(int32_t block_size, int32_t num_heads, int32_t head_size,
                                     gcache_nvfp4_kv_layout* out) {
    if (!out) return GCACHE_ERR_NULL;
    if (block_size <= 0 || num_heads <= 0 || head_size <= 0 || head_size % 16)
        return GCACHE_ERR_SHAPE;
    const int64_t data_row = head_size / 2, scale_row = head_size / 16;
    const int64_t side = (int64_t)block_size * num_heads * (data_row + scale_row);
    out->data_offset = 0;
    out->data_token_stride = data_row;                       // heads outermost
    out->data_head_stride = (int64_t)block_size * data_row;
    out->scale_offset = (int64_t)num_heads * block_size * data_row;
    out->scale_token_stride = scale_row;
    out->scale_head_stride = (int64_t)block_size * scale_row;
    out->side_stride = side;
    out->block_stride = 2 * side;
    return GCACHE_OK;
}

int gcache_reshape_and_cache_nvfp4(const void* key, const void* value, int64_t key_token_stride,
                                   int64_t key_head_stride, int64_t value_token_stride,
                                   int64_t value_head_stride, void* kv_cache,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_heads, int32_t head_size, int64_t num_blocks,
                                   int32_t block_size, const gcache_nvfp4_kv_layout* layout,
                                   const float* k_scale, const float* v_scale,
                                   hipStream_t stream) {
    if (num_tokens < 0) return GCACHE_ERR_SHAPE;
    if (num_tokens == 0) return GCACHE_OK;
    if (!key || !value || !slot_mapping) return GCACHE_ERR_NULL;
    int rc = check_kv(num_heads, head_size, num_blocks, block_size, layout, k_scale, v_scale, kv_cache);
    if (rc) return rc;
    if (!kv_strides_ok(key, key_token_stride, key_head_stride) ||
        !kv_strides_ok(value, value_token_stride, value_head_stride))
        return GCACHE_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    KvWriteParams p;
    p.src[0] = static_cast<const uint16_t*>(key);
    p.src[1] = static_cast<const uint16_t*>(value);
    p.token_stride[0] = key_token_stride;
    p.token_stride[1] = value_token_stride;
    p.head_stride[0] = key_head_stride;
    p.head_stride[1] = value_head_stride;
    p.cache = static_cast<uint8_t*>(kv_cache);
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.num_heads = num_heads;
    p.head_size = head_size;
    p.bph_shift = log2_or_minus1(head_size / 16);
    p.div = make_div(block_size);
    p.L = to_layout(layout);
    p.gscale[0] = k_scale;
    p.gscale[1] = v_scale;
    p.st = staged_layout(p.L, num_heads, head_size);
    return launched(launch_reshape_and_cache_nvfp4(p, stream));
}

int gcache_gather_upconvert_nvfp4_kv(const void* kv_cache, void* key_out, void* value_out,
                                     int64_t total_tokens, int64_t key_token_stride,
                                     int64_t key_head_stride, int64_t value_token_stride,
                                     int64_t value_head_stride, const int32_t* block_table,
                                     int64_t block_table_stride, const int32_t* workspace_starts,
                                     const int32_t* seq_starts, int32_t batch_size,
                                     int32_t num_heads, int32_t head_size, int64_t num_blocks,
                                     int32_t block_size, const gcache_nvfp4_kv_layout* layout,
                                     const float* k_scale, const float* v_scale,
                                     hipStream_t stream) {
    if (total_tokens < 0) return GCACHE_ERR_SHAPE;
    if (total_tokens == 0) return GCACHE_OK;
    if (!key_out || !value_out) return GCACHE_ERR_NULL;
    int rc = check_walk(total_tokens, block_table, block_table_stride, workspace_starts, batch_size);
    if (rc) return rc;
    if ((rc = check_kv(num_heads, head_size, num_blocks, block_size, layout, k_scale, v_scale, kv_cache)))
        return rc;
    if (!kv_strides_ok(key_out, key_token_stride, key_head_stride) ||
        !kv_strides_ok(value_out, value_token_stride, value_head_stride))
        return GCACHE_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    KvGatherParams p;
    p.cache = static_cast<const uint8_t*>(kv_cache);
    p.out[0] = static_cast<uint16_t*>(key_out);
    p.out[1] = static_cast<uint16_t*>(value_out);
    p.token_stride[0] = key_token_stride;
    p.token_stride[1] = value_token_stride;
    p.head_stride[0] = key_head_stride;
    p.head_stride[1] = value_head_stride;
    p.total = total_tokens;
    p.block_table = block_table;
    p.bt_stride = block_table_stride;
    p.ws = workspace_starts;
    p.seq_starts = seq_starts;
    p.batch = batch_size;
    p.num_blocks = num_blocks;
    p.num_heads = num_heads;
    p.head_size = head_size;
    p.cph_shift = log2_or_minus1(head_size / 8);
    p.div = make_div(block_size);
    p.L = to_layout(layout);
    p.gscale[0] = k_scale;
    p.gscale[1] = v_scale;
    p.st = staged_layout(p.L, num_heads, head_size);
    return launched(launch_gather_nvfp4_kv(p, stream));
}

}  // extern "C"
