// gcache_internal.h -- kernel parameter blocks and launchers (host side).
// The extern "C" entry points in gcache_abi.hip validate arguments, then
// fill one of these structs and call the matching launcher.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gcache_device.h"

namespace gcache {

struct DsMlaWriteParams {
    const uint16_t* kv_c;        // bf16 [T, >=512]
    const uint16_t* k_pe;        // bf16 [T, >=64]
    uint8_t* cache;
    const int64_t* slots;        // [T], outside [0, num_slots) = skipped (padding)
    int64_t num_tokens;
    int64_t num_slots;           // num_blocks * block_size
    int64_t kv_c_stride, k_pe_stride;   // elements
    int64_t block_stride, entry_stride; // bytes
    BlockDiv div;                // block_size
};

struct DsMlaGatherParams {
    const uint8_t* cache;
    uint16_t* dst;               // bf16 [total, >=576]
    int64_t total, dst_stride;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* ws;           // workspace_starts [batch]
    const int32_t* seq_starts;   // [batch] or nullptr
    int32_t batch;
    int64_t num_blocks;          // block ids outside [0, num_blocks): zero row
    int64_t block_stride, entry_stride;
    BlockDiv div;
};

struct KvLayout {                // mirrors gcache_nvfp4_kv_layout (bytes)
    int64_t data_offset, data_token_stride, data_head_stride;
    int64_t scale_offset, scale_token_stride, scale_head_stride;
    int64_t side_stride, block_stride;
};

// Staging of the per-head kernels: when the layout keeps a (token, side)'s
// bytes in at most two contiguous, 16-byte aligned runs, the kernels move
// them as 16-byte pieces through an LDS image of `span` bytes per side:
// image bytes [0, run0) are run 0 (at data_offset + off * data_token_stride),
// [run0, span) are run 1 (at scale_offset + off * scale_token_stride).
// Inside the image, head h's data starts at h * data_head and its scales at
// scale_off + h * scale_head.  span == 0: the direct (unstaged) kernels.
struct KvStage {
    int32_t span, run0;
    int32_t data_head, scale_off, scale_head;
};

struct KvWriteParams {
    const uint16_t* src[2];      // key, value: bf16 [T, H, hs]
    int64_t token_stride[2], head_stride[2];  // elements
    uint8_t* cache;
    const int64_t* slots;        // outside [0, num_slots) = skipped
    int64_t num_tokens;
    int64_t num_slots;
    int32_t num_heads, head_size;
    int32_t bph_shift;           // log2(head_size / 16), or -1
    BlockDiv div;
    KvLayout L;
    const float* gscale[2];      // k_scale, v_scale (device scalars)
    KvStage st;                  // st.span > 0: staged kernels
};

struct KvGatherParams {
    const uint8_t* cache;
    uint16_t* out[2];            // key_out, value_out: bf16 [total, H, hs]
    int64_t token_stride[2], head_stride[2];
    int64_t total;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* ws;
    const int32_t* seq_starts;
    int32_t batch;
    int64_t num_blocks;
    int32_t num_heads, head_size;
    int32_t cph_shift;           // log2(head_size / 8), or -1
    BlockDiv div;
    KvLayout L;
    const float* gscale[2];
    KvStage st;                  // st.span > 0: staged kernels
};

struct SparseIndexParams {
    const int32_t* req_id;       // [num_tokens]
    const int32_t* token_indices;// [num_tokens, >=topk], row stride ti_stride
    int32_t* out;                // [num_tokens, >=topk], row stride out_stride
    int64_t num_tokens, ti_stride, out_stride;
    int32_t topk;
    int32_t waves_per_row;       // ceil(topk / indices per wave), set by the launcher
    int32_t vec16;               // 16-byte path allowed
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t batch;
    int64_t num_blocks;
    BlockDiv div;
};

hipError_t launch_write_nvfp4_ds_mla(const DsMlaWriteParams& p, hipStream_t s);
hipError_t launch_write_fp8_ds_mla(const DsMlaWriteParams& p, hipStream_t s);
hipError_t launch_gather_nvfp4_ds_mla(const DsMlaGatherParams& p, hipStream_t s);
hipError_t launch_gather_fp8_ds_mla(const DsMlaGatherParams& p, hipStream_t s);
hipError_t launch_gather_bf16(const DsMlaGatherParams& p, hipStream_t s);
hipError_t launch_reshape_and_cache_nvfp4(const KvWriteParams& p, hipStream_t s);
KvStage staged_layout(const KvLayout& L, int32_t num_heads, int32_t head_size);
hipError_t launch_gather_nvfp4_kv(const KvGatherParams& p, hipStream_t s);
hipError_t launch_convert_req_index(const SparseIndexParams& p, hipStream_t s);

// Events armed by gcache_time_next_launch for the next launch on this host
// thread (consumed by that launch).
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();

// One grid launch.  When timing events are armed, the first piece of the
// launch takes `start` and the last piece `stop` (hipExtLaunchKernel binds
// them to the kernel's own begin and end); otherwise a plain launch.
inline hipError_t launch_piece(const void* kernel, int64_t blocks, int threads, void** args, hipStream_t s,
                               bool first, bool last) {
    LaunchTiming& t = launch_timing();
    hipEvent_t a = first ? t.start : nullptr, b = last ? t.stop : nullptr;
    if (!a && !b) return hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3(threads), args, 0, s);
    if (last) t = LaunchTiming{};
    return hipExtLaunchKernel(kernel, dim3((unsigned)blocks), dim3(threads), args, 0, s, a, b, 0);
}

// Launch `waves` one-shot waves of `kernel(params, wave0)`: the kernel's
// wave index is wave0 + blockIdx.x * kWavesPerBlock + wave_id().  Grids are
// split into launches of at most 2^24 workgroups (far beyond any realistic
// shape); each piece passes its first wave index.
template <typename P>
inline hipError_t launch_waves(void (*kernel)(P, int64_t), int64_t waves, hipStream_t s, const P& p) {
    const int64_t kMaxBlocks = int64_t(1) << 24;
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
        const int64_t nb = blocks - b0 < kMaxBlocks ? blocks - b0 : kMaxBlocks;
        int64_t wave0 = b0 * kWavesPerBlock;
        void* args[] = {const_cast<P*>(&p), &wave0};
        const hipError_t e = launch_piece(reinterpret_cast<const void*>(kernel), nb, kBlockThreads, args, s,
                                          b0 == 0, b0 + nb >= blocks);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Launch `groups` one-shot workgroups of `threads` lanes of
// `kernel(params, group0)`: the kernel's workgroup index is
// group0 + blockIdx.x (pieces of at most 2^24 workgroups, as above).
template <typename P>
inline hipError_t launch_groups(void (*kernel)(P, int64_t), int64_t groups, hipStream_t s, const P& p,
                                int threads = kBlockThreads) {
    const int64_t kMaxBlocks = int64_t(1) << 24;
    for (int64_t b0 = 0; b0 < groups; b0 += kMaxBlocks) {
        const int64_t nb = groups - b0 < kMaxBlocks ? groups - b0 : kMaxBlocks;
        int64_t group0 = b0;
        void* args[] = {const_cast<P*>(&p), &group0};
        const hipError_t e = launch_piece(reinterpret_cast<const void*>(kernel), nb, threads, args, s, b0 == 0,
                                          b0 + nb >= groups);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gcache
