// Measured roofline denominators for the bench: what this GPU sustains for
// a streaming read from HBM and for a bf16 MFMA stream, next to the vendor
// figures (8 TB/s, 2.5 PFLOP/s dense bf16).  Not part of the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Every thread walks 16-byte words of [buf, buf + bytes) with a grid stride,
// UNROLL loads in flight, and folds them with xor; the fold is written only
// under a condition that never holds for the probe's buffer (all zero), so
// the loads stay but nothing is stored.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, size_t words, unsigned *sink)
{
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (UNROLL - 1) * stride < words; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = NT ? __builtin_nontemporal_load(buf + i + u * stride) : buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    for (; i < words; i += stride) acc ^= buf[i];
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[blockIdx.x] = acc[0];
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave;
// 32768 flops per instruction.  Operands come from the (zero-filled) input
// so the compiler cannot fold them; the result is stored only under a
// condition that never holds.
__global__ __launch_bounds__(256) void mfma_stream_kernel(const bf16x8 *in, int iters, float *sink)
{
    const int lane = threadIdx.x & 63;
    const bf16x8 a = in[lane], b = in[64 + lane];
    floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    const float s = c0[0] + c1[1] + c2[2] + c3[3];
    if (s == 123456.75f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int swa_peak_stream_read(const void *buf, size_t bytes, unsigned *sink, int blocks, int unroll, int nt,
                         void *hip_stream)
{
    if (!buf || !sink || blocks < 1 || ((uintptr_t)buf & 15u)) return 1;
    const size_t words = bytes / 16;
    hipStream_t st = (hipStream_t)hip_stream;
    const u32x4 *b = (const u32x4 *)buf;
    if (unroll != 4 && unroll != 8) return 1;
    if (unroll == 4 && nt) hipLaunchKernelGGL((stream_read_kernel<4, true>), dim3(blocks), dim3(256), 0, st, b, words, sink);
    if (unroll == 4 && !nt) hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(blocks), dim3(256), 0, st, b, words, sink);
    if (unroll == 8 && nt) hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(blocks), dim3(256), 0, st, b, words, sink);
    if (unroll == 8 && !nt) hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(blocks), dim3(256), 0, st, b, words, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int swa_peak_mfma(const void *in, float *sink, int blocks, int iters, void *hip_stream)
{
    if (!in || !sink || blocks < 1 || iters < 1 || ((uintptr_t)in & 15u)) return 1;
    hipLaunchKernelGGL(mfma_stream_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream,
                       (const bf16x8 *)in, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
