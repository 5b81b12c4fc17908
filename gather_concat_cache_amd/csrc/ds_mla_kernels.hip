// ds_mla_kernels.hip -- gfx950 kernels for the DS-MLA paged KV cache:
// nvfp4_ds_mla and fp8_ds_mla write, and their gather-upconvert into a
// contiguous bf16 [rows, 576] workspace.
//
// Formats: vLLM PR #51724 digest ("Implementation breakdown" items 2-3, the
// kernel excerpts under "Key source excerpts"); the gather walk with
// seq_starts: vLLM PR #48642 digest ("Implementation breakdown" item 2).
//
// All four kernels are HBM-bound streams with no contraction.  What bounds
// them on MI355X is latency (bytes in flight), the cache state left by the
// previous op and the shape of the write front, so:
//   - every workgroup is one-shot (one small group of tokens or 16 rows,
//     no grid-stride loop): the groups in flight then cover a compact,
//     advancing window of addresses, which the memory system writes far
//     faster than the scattered fronts of persistent loops;
//   - every wave issues all of its loads before it needs them;
//   - every store is a full 16-byte piece: the odd-sized parts of an entry
//     (each lane's NoPE code bytes, scale bytes or fp32 scales, RoPE codes)
//     are assembled in LDS first, so the cache sees whole contiguous runs
//     (up to 1 KiB per store instruction) instead of partial lines written
//     by several instructions;
//   - inputs and outputs use streaming (nontemporal) accesses.
// Mappings:
//   nvfp4 write : one wave per workgroup and two tokens per wave; 8 values
//                 per lane (one 16 B load, one contiguous 1 KiB load per
//                 token); a 16-value block spans two lanes, joined by one
//                 DPP swap.
//   fp8 write   : two waves per workgroup and two tokens per wave; 8 values
//                 per lane (one 16 B load), one token per 64 lanes; the
//                 128-value group amax is a 4-step DPP butterfly inside each
//                 16-lane row.
//   (small workgroups whose staged entries leave in one or two rounds of
//   16-byte stores write faster on MI355X than 16-token groups: measured
//   6.5 vs 6.0 TB/s for both formats at pre-fill sizes.)
//   gathers     : one workgroup per 16 workspace rows; wave 0 resolves the
//                 rows' cache addresses (batch <= 64: workspace_starts held
//                 one per lane and bisected with cross-lane reads, then one
//                 block-table load), the entries are staged in LDS with
//                 16-byte loads, and each row is written by a whole wave
//                 with contiguous 16-byte stores.
#include "gcache_internal.h"

namespace gcache {

// ---------------------------------------------------------------------------
// writes: both formats quantize a group of TILE tokens (TILE / WAVES per
// wave) into an LDS image of their entries, then store the entries as
// 16-byte pieces
// ---------------------------------------------------------------------------
constexpr int kNvWriteWaves = 1, kNvWriteTile = 2;   // nvfp4: 64-lane workgroups, 2 tokens
constexpr int kF8WriteWaves = 2, kF8WriteTile = 4;   // fp8: 128-lane workgroups, 4 tokens

// Cache byte offset of a slot's entry, -1 for a skipped slot.
__device__ __forceinline__ int64_t slot_entry(const DsMlaWriteParams& p, int64_t slot) {
    if (slot < 0) return -1;
    int64_t blk, off;
    split_block(slot, p.div, blk, off);
    return blk * p.block_stride + off * p.entry_stride;
}

// Store the staged entries of the group: piece q = k * EC + j (entry k,
// bytes 16j..16j+15) by thread q mod NT.  Consecutive slots make each
// wave's store one contiguous run of up to 1 KiB.
template <int EB, int TILE, int NT>
__device__ __forceinline__ void store_staged(const DsMlaWriteParams& p, const uint8_t* s_ent,
                                             const int64_t* s_addr) {
    constexpr int EC = EB / 16;
#pragma unroll
    for (int q = threadIdx.x; q < TILE * EC; q += NT) {
        const int k = q / EC;
        const int64_t a = s_addr[k];
        if (a >= 0) st_stream16(p.cache + a + 16 * (q - k * EC), *reinterpret_cast<const uint4*>(s_ent + 16 * q));
    }
}

// Slot ids of tokens t_first + STRIDE*i (-1 past the end or outside the
// cache).  The loads are unconditional -- a token past the end reads the last
// token's id and drops it -- so they are all in flight at once; behind a
// bounds branch each would wait for the one before it (one more memory round
// trip per token before the wave's input loads can start).
template <int N, int STRIDE>
__device__ __forceinline__ void load_slots(const DsMlaWriteParams& p, int64_t t_first, int64_t (&slot)[N]) {
    int64_t raw[N];
#pragma unroll
    for (int i = 0; i < N; i++) {
        const int64_t t = t_first + STRIDE * i;
        raw[i] = p.slots[t < p.num_tokens ? t : p.num_tokens - 1];
    }
#pragma unroll
    for (int i = 0; i < N; i++)
        slot[i] = t_first + STRIDE * i < p.num_tokens ? valid_slot(raw[i], p.num_slots) : -1;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// nvfp4_ds_mla: wave w stages tokens w, w+WAVES, ... of the group, one
// token per 64 lanes: lane l loads NoPE values 8l..8l+7 (one 16 B load, so
// each token is one contiguous 1 KiB load), block l/2's amax joins the two
// halves of the block with one DPP swap of adjacent lanes, both lanes derive
// the same scale and each packs its 4 code bytes.  RoPE: lanes 8i..8i+7
// convert token w+WAVES*i's 64 values, 8 per lane.
template <int WAVES, int TILE>
__global__ __launch_bounds__(WAVES * kWave) void k_write_nvfp4_ds_mla(DsMlaWriteParams p, int64_t group0) {
    constexpr int kTokPerWave = TILE / WAVES;
    static_assert(TILE % WAVES == 0 && kTokPerWave <= 8, "RoPE conversion uses 8 lanes per token");
    __shared__ __align__(16) uint8_t s_ent[TILE * kNvEntry];
    __shared__ int64_t s_addr[TILE];
    const int lane = lane_id(), w = wave_id();
    const int64_t t0 = (group0 + blockIdx.x) * TILE;
    if (t0 >= p.num_tokens) return;                      // workgroup-uniform

    int64_t slot[kTokPerWave];                           // wave-uniform
    uint4 v[kTokPerWave];
    load_slots<kTokPerWave, WAVES>(p, t0 + w, slot);
#pragma unroll
    for (int i = 0; i < kTokPerWave; i++)                // all loads first; padding reads nothing
        if (slot[i] >= 0)
            v[i] = ld_stream16(reinterpret_cast<const uint8_t*>(
                                   p.kv_c + (t0 + w + WAVES * i) * p.kv_c_stride) + 16 * lane);
    const int ri = lane >> 3, rc = lane & 7;
    int64_t rslot = -1;
#pragma unroll
    for (int i = 0; i < kTokPerWave; i++)
        if (ri == i) rslot = slot[i];
    uint4 r = make_uint4(0, 0, 0, 0);
    if (rslot >= 0)
        r = ld_stream16(reinterpret_cast<const uint8_t*>(
                            p.k_pe + (t0 + w + WAVES * ri) * p.k_pe_stride) + 16 * rc);

#pragma unroll
    for (int i = 0; i < kTokPerWave; i++) {
        const int k = w + WAVES * i;
        if (lane == 0) s_addr[k] = slot_entry(p, slot[i]);
        if (slot[i] < 0) continue;                       // wave-uniform: DPP below sees all lanes
        const uint32_t wv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float x[8];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            x[2 * q] = bf16_lo(wv[q]);
            x[2 * q + 1] = bf16_hi(wv[q]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; q++) amax = fmaxf(amax, fabsf(x[q]));
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));    // quad_perm [1,0,3,2]: the other half of the block
        // Block scale: e4m3_rn_sat(amax / 6), then the binary32 reciprocal
        // of its decoded value (0 for a zero scale).
        const uint32_t sf = put_e4m3x2<false>(0u, amax / 6.0f, 0.0f) & 0xFFu;
        const float s = e4m3_f32(sf);
        const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
        uint32_t q0 = 0;
        q0 = put_e2m1x2<0>(q0, x[0] * inv, x[1] * inv);
        q0 = put_e2m1x2<1>(q0, x[2] * inv, x[3] * inv);
        q0 = put_e2m1x2<2>(q0, x[4] * inv, x[5] * inv);
        q0 = put_e2m1x2<3>(q0, x[6] * inv, x[7] * inv);
        uint8_t* e = s_ent + k * kNvEntry;
        *reinterpret_cast<uint32_t*>(e + 4 * lane) = q0;
        if ((lane & 1) == 0) e[kNvScaleOff + (lane >> 1)] = (uint8_t)sf;
    }
    if (rslot >= 0) {                                    // RoPE values 8rc..8rc+7 -> 8 e4m3 bytes
        uint32_t a = 0, b = 0;
        a = put_e4m3x2<false>(a, bf16_lo(r.x), bf16_hi(r.x));
        a = put_e4m3x2<true>(a, bf16_lo(r.y), bf16_hi(r.y));
        b = put_e4m3x2<false>(b, bf16_lo(r.z), bf16_hi(r.z));
        b = put_e4m3x2<true>(b, bf16_lo(r.w), bf16_hi(r.w));
        *reinterpret_cast<uint2*>(s_ent + (w + WAVES * ri) * kNvEntry + kNvRopeOff + 8 * rc) =
            make_uint2(a, b);
    }
    __syncthreads();
    store_staged<kNvEntry, TILE, WAVES * kWave>(p, s_ent, s_addr);
}

// fp8_ds_mla: 512 e4m3 | 4 x fp32 scale (amax / 448 per 128) | 64 bf16.
// Wave w stages tokens w, w+WAVES, ... of the group, one token per 64 lanes
// (8 values per lane); the 128-value group amax is a 4-step DPP butterfly
// inside each 16-lane row.  RoPE: lanes 8i..8i+7 copy token w+WAVES*i's
// 128 B.
template <int WAVES, int TILE>
__global__ __launch_bounds__(WAVES * kWave) void k_write_fp8_ds_mla(DsMlaWriteParams p, int64_t group0) {
    constexpr int kTokPerWave = TILE / WAVES;
    static_assert(TILE % WAVES == 0 && kTokPerWave <= 8, "RoPE copy uses 8 lanes per token");
    __shared__ __align__(16) uint8_t s_ent[TILE * kF8Entry];
    __shared__ int64_t s_addr[TILE];
    const int lane = lane_id(), w = wave_id();
    const int64_t t0 = (group0 + blockIdx.x) * TILE;
    if (t0 >= p.num_tokens) return;                      // workgroup-uniform

    int64_t slot[kTokPerWave];                           // wave-uniform
    uint4 v[kTokPerWave];
    load_slots<kTokPerWave, WAVES>(p, t0 + w, slot);
#pragma unroll
    for (int i = 0; i < kTokPerWave; i++)
        if (slot[i] >= 0)
            v[i] = ld_stream16(reinterpret_cast<const uint8_t*>(
                                   p.kv_c + (t0 + w + WAVES * i) * p.kv_c_stride) + 16 * lane);
    const int ri = lane >> 3, rc = lane & 7;
    int64_t rslot = -1;
#pragma unroll
    for (int i = 0; i < kTokPerWave; i++)
        if (ri == i) rslot = slot[i];
    uint4 r = make_uint4(0, 0, 0, 0);
    if (rslot >= 0)
        r = ld_stream16(reinterpret_cast<const uint8_t*>(
                            p.k_pe + (t0 + w + WAVES * ri) * p.k_pe_stride) + 16 * rc);

#pragma unroll
    for (int i = 0; i < kTokPerWave; i++) {
        const int k = w + WAVES * i;
        if (lane == 0) s_addr[k] = slot_entry(p, slot[i]);
        if (slot[i] < 0) continue;                       // wave-uniform: DPP below sees all lanes
        const uint32_t wv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float x[8];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            x[2 * q] = bf16_lo(wv[q]);
            x[2 * q + 1] = bf16_hi(wv[q]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; q++) amax = fmaxf(amax, fabsf(x[q]));
        // 16 lanes x 8 values = one 128-value group: butterfly max in the row.
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));    // quad_perm [1,0,3,2]
        amax = fmaxf(amax, dpp_f32<0x4E>(amax));    // quad_perm [2,3,0,1]
        amax = fmaxf(amax, dpp_f32<0x141>(amax));   // row_half_mirror
        amax = fmaxf(amax, dpp_f32<0x140>(amax));   // row_mirror
        const float sc = amax / 448.0f;
        const float inv = (sc == 0.0f) ? 0.0f : 1.0f / sc;
        uint32_t q0 = 0, q1 = 0;
        q0 = put_e4m3x2<false>(q0, x[0] * inv, x[1] * inv);
        q0 = put_e4m3x2<true>(q0, x[2] * inv, x[3] * inv);
        q1 = put_e4m3x2<false>(q1, x[4] * inv, x[5] * inv);
        q1 = put_e4m3x2<true>(q1, x[6] * inv, x[7] * inv);
        uint8_t* e = s_ent + k * kF8Entry;
        *reinterpret_cast<uint2*>(e + 8 * lane) = make_uint2(q0, q1);
        if ((lane & 15) == 0) *reinterpret_cast<float*>(e + kF8ScaleOff + 4 * (lane >> 4)) = sc;
    }
    if (rslot >= 0)
        *reinterpret_cast<uint4*>(s_ent + (w + WAVES * ri) * kF8Entry + kF8RopeOff + 16 * rc) = r;
    __syncthreads();
    store_staged<kF8Entry, TILE, WAVES * kWave>(p, s_ent, s_addr);
}

// ---------------------------------------------------------------------------
// gathers
// ---------------------------------------------------------------------------
constexpr int kGatherTile = 16;    // workspace rows per workgroup

// Wave 0 resolves the cache offsets of rows r0 .. r0+nrows-1 (lane i: row
// r0+i); -1 marks a row whose walk leaves the block table or the cache.
__device__ __forceinline__ int64_t tile_row_entry(const DsMlaGatherParams& p, int64_t r0, int nrows,
                                                  int lane) {
    const int64_t r = r0 + lane;
    int b = 0;
    int64_t ws_b = 0, ss_b = 0;
    if (p.batch <= kWave) {
        // one load of workspace_starts / seq_starts per lane, then a
        // bisection by cross-lane reads: no dependent global loads
        const bool in = lane < p.batch;
        const int32_t wsl = in ? p.ws[lane] : 0x7FFFFFFF;
        const int32_t ssl = (in && p.seq_starts) ? p.seq_starts[lane] : 0;
        b = bisect_request64([&](int i) { return (int64_t)__shfl(wsl, i); }, p.batch, r);
        ws_b = __shfl(wsl, b);
        ss_b = __shfl(ssl, b);
    } else if (lane < nrows) {
        b = find_request(p.ws, p.batch, r, p.total);
        ws_b = p.ws[b];
        ss_b = p.seq_starts ? p.seq_starts[b] : 0;
    }
    if (lane >= nrows) return -1;
    return row_entry(p.block_table, p.bt_stride, b, ws_b, ss_b, r, p.div, p.num_blocks, p.block_stride,
                     p.entry_stride);
}

// One workgroup per tile of kGatherTile consecutive workspace rows:
//   1. wave 0 resolves the rows' entry offsets into LDS;
//   2. every 16-byte piece of the tile's entries is loaded (all loads in
//      flight before any is stored) and staged in LDS;
//   3. each wave converts and stores whole NoPE rows (64 lanes x 16 B), then
//      the RoPE pieces (8 x 16 B per row) are spread over the workgroup.
// Rows with an invalid walk are written as zeros.
template <bool NVFP4>
__global__ __launch_bounds__(kBlockThreads) void k_gather_ds_mla(DsMlaGatherParams p, int64_t tile0) {
    constexpr int EB = NVFP4 ? kNvEntry : kF8Entry;      // entry bytes used
    constexpr int EC = EB / 16;                          // 16-byte pieces per entry
    constexpr int kPieces = (kGatherTile * EC + kBlockThreads - 1) / kBlockThreads;
    __shared__ __align__(16) uint8_t s_ent[kGatherTile * EB];
    __shared__ int64_t s_off[kGatherTile];

    const int tid = threadIdx.x;
    const int64_t r0 = (tile0 + blockIdx.x) * kGatherTile;
    if (r0 >= p.total) return;                           // workgroup-uniform
    const int nrows = (int)min((int64_t)kGatherTile, p.total - r0);
    if (tid < kWave) {
        const int64_t e = tile_row_entry(p, r0, nrows, tid);
        if (tid < kGatherTile) s_off[tid] = e;
    }
    __syncthreads();

    uint4 v[kPieces];
#pragma unroll
    for (int k = 0; k < kPieces; k++) {
        const int j = tid + kBlockThreads * k;
        const int row = j / EC;
        if (j < kGatherTile * EC && row < nrows && s_off[row] >= 0)
            v[k] = ld_stream16(p.cache + s_off[row] + 16 * (j - row * EC));
    }
#pragma unroll
    for (int k = 0; k < kPieces; k++) {
        const int j = tid + kBlockThreads * k;
        const int row = j / EC;
        if (j < kGatherTile * EC && row < nrows && s_off[row] >= 0)
            *reinterpret_cast<uint4*>(s_ent + 16 * j) = v[k];
    }
    __syncthreads();

    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < kGatherTile / kWavesPerBlock; i++) {
        const int row = w + kWavesPerBlock * i;
        if (row >= nrows) break;
        const uint8_t* e = s_ent + row * EB;
        uint4 o = make_uint4(0, 0, 0, 0);
        if (s_off[row] >= 0) {
            if (NVFP4) {                                 // values 8l..8l+7, block l/2
                const uint32_t nib = *reinterpret_cast<const uint32_t*>(e + 4 * lane);
                const float s = e4m3_f32(e[kNvScaleOff + (lane >> 1)]);
                const f32x2 a = e2m1x2_f32<0>(nib), b = e2m1x2_f32<1>(nib);
                const f32x2 c = e2m1x2_f32<2>(nib), d = e2m1x2_f32<3>(nib);
                o = make_uint4(pack_bf16x2(a.x * s, a.y * s), pack_bf16x2(b.x * s, b.y * s),
                               pack_bf16x2(c.x * s, c.y * s), pack_bf16x2(d.x * s, d.y * s));
            } else {                                     // values 8l..8l+7, group l/16
                const uint2 q = *reinterpret_cast<const uint2*>(e + 8 * lane);
                const float sc = *reinterpret_cast<const float*>(e + kF8ScaleOff + 4 * (lane >> 4));
                const f32x2 a = e4m3x2_f32<false>(q.x), b = e4m3x2_f32<true>(q.x);
                const f32x2 c = e4m3x2_f32<false>(q.y), d = e4m3x2_f32<true>(q.y);
                o = make_uint4(pack_bf16x2(a.x * sc, a.y * sc), pack_bf16x2(b.x * sc, b.y * sc),
                               pack_bf16x2(c.x * sc, c.y * sc), pack_bf16x2(d.x * sc, d.y * sc));
            }
        }
        st_stream16(p.dst + (r0 + row) * p.dst_stride + 8 * lane, o);
    }
    if (tid < nrows * 8) {                               // RoPE: 8 pieces of 8 values per row
        const int row = tid >> 3, c = tid & 7;
        const uint8_t* e = s_ent + row * EB;
        uint4 o = make_uint4(0, 0, 0, 0);
        if (s_off[row] >= 0) {
            if (NVFP4) {
                const uint2 q = *reinterpret_cast<const uint2*>(e + kNvRopeOff + 8 * c);
                const f32x2 a = e4m3x2_f32<false>(q.x), b = e4m3x2_f32<true>(q.x);
                const f32x2 cc = e4m3x2_f32<false>(q.y), d = e4m3x2_f32<true>(q.y);
                o = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y), pack_bf16x2(cc.x, cc.y),
                               pack_bf16x2(d.x, d.y));
            } else {
                o = *reinterpret_cast<const uint4*>(e + kF8RopeOff + 16 * c);
            }
        }
        st_stream16(p.dst + (r0 + row) * p.dst_stride + kNope + 8 * c, o);
    }
}

// BF16 comparator: the same tile walk over a cache whose 1152-byte entries
// hold the row's 576 bf16 values; each 16-byte piece is copied straight from
// the cache to the workspace (all loads of the tile first, no LDS).
constexpr int kBf16Entry = 2 * (kNope + kRope);
constexpr int kBf16Pieces = kBf16Entry / 16;           // 72 per row

__global__ __launch_bounds__(kBlockThreads) void k_gather_bf16(DsMlaGatherParams p, int64_t tile0) {
    constexpr int kPieces = (kGatherTile * kBf16Pieces + kBlockThreads - 1) / kBlockThreads;
    __shared__ int64_t s_off[kGatherTile];
    const int tid = threadIdx.x;
    const int64_t r0 = (tile0 + blockIdx.x) * kGatherTile;
    if (r0 >= p.total) return;                           // workgroup-uniform
    const int nrows = (int)min((int64_t)kGatherTile, p.total - r0);
    if (tid < kWave) {
        const int64_t e = tile_row_entry(p, r0, nrows, tid);
        if (tid < kGatherTile) s_off[tid] = e;
    }
    __syncthreads();
    uint4 v[kPieces];
#pragma unroll
    for (int k = 0; k < kPieces; k++) {
        const int j = tid + kBlockThreads * k;
        const int row = j / kBf16Pieces;
        v[k] = make_uint4(0, 0, 0, 0);
        if (j < kGatherTile * kBf16Pieces && row < nrows && s_off[row] >= 0)
            v[k] = ld_stream16(p.cache + s_off[row] + 16 * (j - row * kBf16Pieces));
    }
#pragma unroll
    for (int k = 0; k < kPieces; k++) {
        const int j = tid + kBlockThreads * k;
        const int row = j / kBf16Pieces;
        if (j < kGatherTile * kBf16Pieces && row < nrows)
            st_stream16(p.dst + (r0 + row) * p.dst_stride + 8 * (j - row * kBf16Pieces), v[k]);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_write_nvfp4_ds_mla(const DsMlaWriteParams& p, hipStream_t s) {
    return launch_groups(k_write_nvfp4_ds_mla<kNvWriteWaves, kNvWriteTile>,
                         (p.num_tokens + kNvWriteTile - 1) / kNvWriteTile, s, p, kNvWriteWaves * kWave);
}
hipError_t launch_write_fp8_ds_mla(const DsMlaWriteParams& p, hipStream_t s) {
    return launch_groups(k_write_fp8_ds_mla<kF8WriteWaves, kF8WriteTile>,
                         (p.num_tokens + kF8WriteTile - 1) / kF8WriteTile, s, p, kF8WriteWaves * kWave);
}
hipError_t launch_gather_nvfp4_ds_mla(const DsMlaGatherParams& p, hipStream_t s) {
    return launch_groups(k_gather_ds_mla<true>, (p.total + kGatherTile - 1) / kGatherTile, s, p);
}
hipError_t launch_gather_fp8_ds_mla(const DsMlaGatherParams& p, hipStream_t s) {
    return launch_groups(k_gather_ds_mla<false>, (p.total + kGatherTile - 1) / kGatherTile, s, p);
}
hipError_t launch_gather_bf16(const DsMlaGatherParams& p, hipStream_t s) {
    return launch_groups(k_gather_bf16, (p.total + kGatherTile - 1) / kGatherTile, s, p);
}

}  // namespace gcache
