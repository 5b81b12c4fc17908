// converter_sweep.hip -- test-only gfx950 kernels that run the library's
// device conversion helpers (gcache_device.h) and the binary32 divisions the
// kernels perform, over caller-chosen inputs, so that a host comparator can
// check every result against the CPU oracle's encoders and C arithmetic.
//
// What the kernels of libgcache.so compute with these helpers:
//   put_e2m1x2<SEL>  e2m1 codes of x * inv            (NVFP4 writes)
//   put_e4m3x2<HI>   e4m3 codes of amax / 6, (amax / 6) / gs, x * inv and
//                    the RoPE values                  (all writes)
//   pack_bf16x2      bf16 of the dequantized products (all gathers)
//   e2m1x2_f32, e4m3x2_f32, e4m3_f32: decoders        (gathers, writes)
//   amax / 6.0f, amax / 448.0f, 1.0f / s, (amax / 6.0f) / gs
// Built with the library's own flags (no fast-math, -ffp-contract=off).
// Nothing here is part of the library; only the GPU tests load it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../gather_concat_cache_amd/csrc/gcache_device.h"

using namespace gcache;

namespace {

// Thread i takes the four binary32 patterns base + 4i .. base + 4i + 3.
//   fp4[i]   bytes 0, 1: put_e2m1x2<0>, <1> of (x0, x1), (x2, x3);
//            bytes 2, 3: put_e2m1x2<2>, <3> of the same pairs
//   fp8[i]   put_e4m3x2<false> of (x0, x1), put_e4m3x2<true> of (x2, x3)
//   bf16[i]  pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)
//   div6, div448, recip: x / 6, x / 448, 1 / x for x0..x3
__global__ __launch_bounds__(256) void k_sweep_unary(uint32_t base, uint32_t n4, uint32_t* fp4, uint32_t* fp8,
                                                     uint2* bf16, uint4* div6, uint4* div448, uint4* recip) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n4) return;
    const uint32_t u = base + 4u * i;
    const float x0 = __uint_as_float(u), x1 = __uint_as_float(u + 1u);
    const float x2 = __uint_as_float(u + 2u), x3 = __uint_as_float(u + 3u);
    uint32_t q = 0;
    q = put_e2m1x2<0>(q, x0, x1);
    q = put_e2m1x2<1>(q, x2, x3);
    q = put_e2m1x2<2>(q, x0, x1);
    q = put_e2m1x2<3>(q, x2, x3);
    fp4[i] = q;
    uint32_t c = 0;
    c = put_e4m3x2<false>(c, x0, x1);
    c = put_e4m3x2<true>(c, x2, x3);
    fp8[i] = c;
    bf16[i] = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
    div6[i] = make_uint4(__float_as_uint(x0 / 6.0f), __float_as_uint(x1 / 6.0f), __float_as_uint(x2 / 6.0f),
                         __float_as_uint(x3 / 6.0f));
    div448[i] = make_uint4(__float_as_uint(x0 / 448.0f), __float_as_uint(x1 / 448.0f),
                           __float_as_uint(x2 / 448.0f), __float_as_uint(x3 / 448.0f));
    recip[i] = make_uint4(__float_as_uint(1.0f / x0), __float_as_uint(1.0f / x1), __float_as_uint(1.0f / x2),
                          __float_as_uint(1.0f / x3));
}

// q[i] = (a[i] / 6) / b[i], the per-head scale argument.
__global__ __launch_bounds__(256) void k_sweep_scale_div(const float* a, const float* b, uint32_t* q, uint32_t n) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    q[i] = __float_as_uint((a[i] / 6.0f) / b[i]);
}

// Decoders over every code.  Thread c (0..255):
//   e4m3[4c + k]: e4m3x2_f32<false>, <true> of the word (c | c << 8 | c << 16
//                 | c << 24): both halves of both words, plus e4m3_f32(c)
//   e2m1[8c + k]: e2m1x2_f32<SEL> of the byte c in every position SEL
__global__ __launch_bounds__(256) void k_sweep_decoders(float* e4m3, float* e2m1) {
    const uint32_t c = threadIdx.x;
    const uint32_t w = c | (c << 8) | (c << 16) | (c << 24);
    const f32x2 lo = e4m3x2_f32<false>(w), hi = e4m3x2_f32<true>(w);
    e4m3[5 * c + 0] = lo.x;
    e4m3[5 * c + 1] = lo.y;
    e4m3[5 * c + 2] = hi.x;
    e4m3[5 * c + 3] = hi.y;
    e4m3[5 * c + 4] = e4m3_f32(c);
    const f32x2 a = e2m1x2_f32<0>(w), b = e2m1x2_f32<1>(w), d = e2m1x2_f32<2>(w), e = e2m1x2_f32<3>(w);
    e2m1[8 * c + 0] = a.x;
    e2m1[8 * c + 1] = a.y;
    e2m1[8 * c + 2] = b.x;
    e2m1[8 * c + 3] = b.y;
    e2m1[8 * c + 4] = d.x;
    e2m1[8 * c + 5] = d.y;
    e2m1[8 * c + 6] = e.x;
    e2m1[8 * c + 7] = e.y;
}

}  // namespace

// Host launchers (device pointers; count a multiple of 4 for the unary sweep).
extern "C" int sweep_unary(uint32_t base, uint32_t count, void* fp4, void* fp8, void* bf16, void* div6,
                           void* div448, void* recip, hipStream_t s) {
    if (count % 4u) return -1;
    const uint32_t n4 = count / 4u;
    hipLaunchKernelGGL(k_sweep_unary, dim3((n4 + 255u) / 256u), dim3(256), 0, s, base, n4,
                       static_cast<uint32_t*>(fp4), static_cast<uint32_t*>(fp8), static_cast<uint2*>(bf16),
                       static_cast<uint4*>(div6), static_cast<uint4*>(div448), static_cast<uint4*>(recip));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int sweep_scale_div(const void* a, const void* b, void* q, uint32_t n, hipStream_t s) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_sweep_scale_div, dim3((n + 255u) / 256u), dim3(256), 0, s,
                       static_cast<const float*>(a), static_cast<const float*>(b), static_cast<uint32_t*>(q), n);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int sweep_decoders(void* e4m3, void* e2m1, hipStream_t s) {
    hipLaunchKernelGGL(k_sweep_decoders, dim3(1), dim3(256), 0, s, static_cast<float*>(e4m3),
                       static_cast<float*>(e2m1));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
