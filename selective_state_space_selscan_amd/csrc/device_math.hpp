// Device-side scalar helpers for the gfx950 selective-scan kernels:
// bf16 <-> fp32 conversion, softplus, SiLU and the hardware exp2/log2/rcp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace selscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7fffffffu) > 0x7f800000u)
        return (x >> 16) | 0x40u;
    x += 0x7fffu + ((x >> 16) & 1u);
    return x >> 16;
}

// Element access for the two storage types (float, or bf16 held as uint16_t).
__device__ __forceinline__ float load_elem(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ void store_elem(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t *p, int64_t i, float v) {
    p[i] = (uint16_t)f32_to_bf16_bits(v);
}

// Hardware transcendental instructions (v_exp_f32 = 2^x, v_log_f32 = log2 x,
// v_rcp_f32 = 1/x), each accurate to about 1 ulp.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 2^x for the decay of one step, x = Delta A log2(e) <= 0, with fp32-level
// accuracy where it matters.  v_exp_f32 is accurate to about 1 ulp, but its
// errors do not average out: when 2^x is close to 1 (a slow decay, small
// Delta |A|) the product of many steps' decays, which a state carries for
// about 1 / (Delta |A|) steps, picks up their sum (measured: a 1e-4 error in
// y after 96 steps of an fp32 sequence whose initial state decays slowly).
// For |x| < 1/16 the Taylor series of 2^x - 1 in x (degree 5, truncation
// below 1e-10 relative) is added to 1, one rounding to nearest; elsewhere the
// hardware exp2 is used (1 - 2^x > 0.04 there, so an ulp of 2^x is small
// against the decay it describes).
__device__ __forceinline__ float exp2_decay_accurate(float x) {
    constexpr float c1 = kLn2;
    constexpr float c2 = kLn2 * kLn2 / 2.0f;
    constexpr float c3 = kLn2 * kLn2 * kLn2 / 6.0f;
    constexpr float c4 = kLn2 * kLn2 * kLn2 * kLn2 / 24.0f;
    constexpr float c5 = kLn2 * kLn2 * kLn2 * kLn2 * kLn2 / 120.0f;
    const float p = fmaf(x, fmaf(x, fmaf(x, fmaf(x, c5, c4), c3), c2), c1);
    const float series = fmaf(x, p, 1.0f);
    return fabsf(x) < 0.0625f ? series : hw_exp2(x);
}

// The step decay for the storage type: fp32 inputs are held to a 1e-4
// relative tolerance, which needs exp2_decay_accurate; bf16 inputs (5e-3) use
// the hardware exp2 directly.
__device__ __forceinline__ float exp2_decay(float x, const float *) { return exp2_decay_accurate(x); }
__device__ __forceinline__ float exp2_decay(float x, const uint16_t *) { return hw_exp2(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
// log1p(w) for w in (0, 1]: s = fl(1 + w) loses the low bits of w, so the
// rounding error c = w - (s - 1) (exact, Fast2Sum) is added back:
// log(1 + w) = log(s) + log(1 + c/s) ~= log(s) + c, an error below 2^-24 relative.
__device__ __forceinline__ float softplus(float x) {
    float w = hw_exp2(-fabsf(x) * kLog2e);
    float s = 1.0f + w;
    float c = w - (s - 1.0f);
    float lp = fmaf(hw_log2(s), kLn2, c);
    return fmaxf(x, 0.0f) + lp;
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu(float z) {
    return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

} // namespace selscan
