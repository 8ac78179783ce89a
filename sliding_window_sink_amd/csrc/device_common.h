// Device helpers shared by the gfx950 kernels: vector types, bf16 <-> fp32,
// MFMA wrappers and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 operands along the MFMA contraction held by one lane: bf16x8 (16 bytes)
// for bf16 data, floatx8 (32 bytes) for fp32 data.
template <typename T> struct Frag;
template <> struct Frag<bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = floatx8; };

// c += A * B for one 16x16 output tile with a 32-deep contraction.  Lane l
// supplies row/column l%16 and contraction indices 8*(l/16) .. 8*(l/16)+7 of
// both operands; the result layout is rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ floatx4 mma16x16x32(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 variant: eight 16x16x4 MFMAs.  In MFMA j, lane group g = l/16 feeds
// contraction index g, which carries element j of the lane's 8 -- so over the
// eight MFMAs every lane's 8 elements are consumed exactly once and the sum is
// the same 32-deep contraction as above.
__device__ __forceinline__ floatx4 mma16x16x32(floatx8 a, floatx8 b, floatx4 c)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

// c += A * B for one 32x32 output tile with a 16-deep contraction.  Lane l
// supplies row/column l%32 and contraction indices 8*(l/32) .. 8*(l/32)+7 of
// both operands; element 4*j+i of the result is row 8*j + 4*(l/32) + i,
// column l%32.
__device__ __forceinline__ floatx16 mma32x32x16(bf16x8 a, bf16x8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 variant: eight 32x32x2 MFMAs; in MFMA j lane group l/32 feeds
// contraction index l/32 carrying element j of the lane's 8 (same sum).
__device__ __forceinline__ floatx16 mma32x32x16(floatx8 a, floatx8 b, floatx16 c)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

// Fragment loads at 16-byte granularity (the buffers are only 16-B aligned).
template <typename F> __device__ __forceinline__ F load_frag(const void *p);
template <> __device__ __forceinline__ bf16x8 load_frag<bf16x8>(const void *p)
{
    return *(const bf16x8 *)p;
}
template <> __device__ __forceinline__ floatx8 load_frag<floatx8>(const void *p)
{
    const floatx4 a = ((const floatx4 *)p)[0], b = ((const floatx4 *)p)[1];
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename F> __device__ __forceinline__ F to_frag(const float (&v)[8]);
template <> __device__ __forceinline__ bf16x8 to_frag<bf16x8>(const float (&v)[8])
{
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];
    return r;
}
template <> __device__ __forceinline__ floatx8 to_frag<floatx8>(const float (&v)[8])
{
    floatx8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = v[j];
    return r;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask)
{
    return fmaxf(v, __shfl_xor(v, mask, 64));
}

// Raw buffer resource over [base, base + nbytes): loads at offsets past the
// end return zero.  The descriptor lives in scalar registers.
constexpr int kBufferConfig = 0x00020000;  // gfx9 data format field; no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, kBufferConfig);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}
// Cache-policy bits of a buffer load: nt (non-temporal) marks the lines as
// streamed, to be replaced first.  Data read once per launch (a decode
// step's K/V cache) takes it; a streaming read of 128 MiB ran 8 % faster with
// it on this GPU.
constexpr int kPolicyNT = 2;
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, int byte_offset)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kPolicyNT));
}

// Map the hardware workgroup id onto a logical tile id so that the workgroups
// an XCD receives (ids congruent mod 8) cover consecutive logical tiles; the
// tail that does not divide by 8 keeps its own ids.
__device__ __forceinline__ int xcd_remap(int hw, int total)
{
    const int per = total >> 3;
    if (hw < (per << 3)) return (hw & 7) * per + (hw >> 3);
    return hw;
}

}  // namespace swa
