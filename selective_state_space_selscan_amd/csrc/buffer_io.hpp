// Memory-access helpers shared by the forward kernels: raw buffer loads and
// stores with scalar descriptors, and scalar (SGPR) reads of wave-uniform rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.hpp"

namespace selscan {

// Raw buffer access (MUBUF) with a per-segment descriptor: the base address
// and byte range are scalar, the per-lane offset is lane * sizeof(element), and
// the per-timestep offset is a scalar, so no VALU goes into addressing.  Loads
// past the range return 0 and stores past it are dropped, which covers the
// ragged end of the sequence.  Word 3 = 0x00020000 is the gfx9-family raw
// buffer format (32-bit data format).
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int nrec = bytes > 0 ? (int)bytes : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nrec, kBufWord3);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float *)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, const uint16_t *)
{
    return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v, float *)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int voff, int soff, float v, uint16_t *)
{
    // v_cvt_pk_bf16_f32: round to nearest even, NaN preserved
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, voff, soff, 0);
}

// Wave-uniform data (B_t, C_t rows or columns) is read through the constant
// address space, so that the reads become scalar loads (s_load_dwordxN) into
// SGPRs even across barriers.  The data must not change during the kernel.
typedef __attribute__((address_space(4))) const float const_f32;
typedef __attribute__((address_space(4))) const uint32_t const_u32;
__device__ __forceinline__ const const_f32 *as_const(const float *p)
{
    return (const const_f32 *)(uintptr_t)p;
}
__device__ __forceinline__ const const_u32 *as_const_u32(const void *p)
{
    return (const const_u32 *)(uintptr_t)p;
}

// Overload tag for the element type (float, or bf16 held as uint16_t).
template <typename T>
__device__ __forceinline__ const T *tag()
{
    return (const T *)nullptr;
}

// Element loads that keep the fp32 bit pattern in a uint32_t (held in the
// prefetch buffers, turned into a float with raw_to_f32 at the point of use):
// an fp32 value as loaded; a bf16 value shifted into the top half (its fp32
// pattern) right at the load.  Shifting there, where the compiler sees the
// 16-bit load's zero extension, takes one instruction; shifting at the use,
// across the prefetch loop, took a mask and a shift per element.
__device__ __forceinline__ uint32_t buf_load_raw(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 const float *)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load_raw(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 const uint16_t *)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0) << 16;
}
__device__ __forceinline__ float raw_to_f32(uint32_t v, const float *) { return __uint_as_float(v); }
__device__ __forceinline__ float raw_to_f32(uint32_t v, const uint16_t *) { return __uint_as_float(v); }

// One row of N values (N even) shared by the whole wave, as scalar loads.
template <int N>
__device__ __forceinline__ void load_row(const float *p, int64_t row, float (&v)[N])
{
    const const_f32 *q = as_const(p) + row * N;
#pragma unroll
    for (int n = 0; n < N; ++n)
        v[n] = q[n];
}
template <int N>
__device__ __forceinline__ void load_row(const uint16_t *p, int64_t row, float (&v)[N])
{
    const const_u32 *q = as_const_u32(p) + row * (N / 2);
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
        const uint32_t w = q[k];
        v[2 * k] = __uint_as_float(w << 16);
        v[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
    }
}


} // namespace selscan
