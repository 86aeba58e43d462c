// Decode step for gfx950: one t-step of the selective recurrence applied in
// place to a resident fp32 state (batch, dim, N).
//
// Decode keeps one fixed-size state per sample and does O(1) work per token
// (Mamba tutorial, pwwt.cn, §5.1 table and §6.3).  The paper walkthrough
// (m.lqnn.cn) §3.2 names this single-token state update.  The step is
// HBM-bound: each state entry is read once and written once, 8 bytes per
// (b, d, n), against a handful of flops.
//
// Layout of the work: N/4 consecutive lanes share one (b, d) row of N states,
// each lane owning one float4 of it, so every state load or store instruction
// of a wave covers 1 KB of contiguous memory.  Each lane updates its 4 states,
// forms its part of C.h, and the row's lanes sum the parts with xor-shuffles.
// The per-row scalars (Delta, u, z) are recomputed by every lane of the row,
// which costs nothing measurable in a memory-bound step.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace {

constexpr int kBlock = 256;

template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&v)[4]);

template <>
__device__ __forceinline__ void load4<float>(const float *p, float (&v)[4])
{
    const float4 x = *reinterpret_cast<const float4 *>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t *p, float (&v)[4])
{
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(x.x << 16);
    v[1] = __uint_as_float(x.x & 0xffff0000u);
    v[2] = __uint_as_float(x.y << 16);
    v[3] = __uint_as_float(x.y & 0xffff0000u);
}

template <int N, typename T>
__global__ __launch_bounds__(kBlock) void state_update_kernel(
    float *__restrict__ state, const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D_skip, const T *__restrict__ z,
    const float *__restrict__ delta_bias, int delta_softplus, T *__restrict__ y, int64_t dim,
    int64_t rows)
{
    static_assert(N % 4 == 0 && kBlock % (N / 4) == 0, "N/4 lanes per row");
    constexpr int R = N / 4;                       // lanes per (b, d) row
    const int64_t gt = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t row = gt / R;
    const int q = (int)(gt % R);                   // this lane's float4 of the row
    const bool valid = row < rows;
    const int64_t r = valid ? row : rows - 1;      // tail lanes compute on a valid row
    const int64_t b = r / dim;
    const int64_t d = r - b * dim;

    float4 *srow = reinterpret_cast<float4 *>(state + r * N) + q;
    const float4 h4 = *srow;
    const float4 a4 = *reinterpret_cast<const float4 *>(A + d * N + 4 * q);
    float Bv[4], Cv[4];
    load4<T>(Bm + b * N + 4 * q, Bv);
    load4<T>(Cm + b * N + 4 * q, Cv);

    const float ut = load_elem(u, r);
    const float x = load_elem(delta, r) + (delta_bias ? delta_bias[d] : 0.0f);
    const float dt = delta_softplus ? softplus(x) : x;
    const float du = dt * ut;
    const float dA = dt * kLog2e;
    float h[4] = {h4.x, h4.y, h4.z, h4.w};
    const float a[4] = {a4.x, a4.y, a4.z, a4.w};
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[k] = fmaf(hw_exp2(dA * a[k]), h[k], du * Bv[k]);
        acc = fmaf(Cv[k], h[k], acc);
    }
    // sum C.h over the R lanes of the row (all lanes take part)
#pragma unroll
    for (int off = R / 2; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off, R);
    if (valid) {
        *srow = make_float4(h[0], h[1], h[2], h[3]);
        if (q == 0) {
            float yv = fmaf(D_skip ? D_skip[d] : 0.0f, ut, acc);
            if (z)
                yv *= silu(load_elem(z, r));
            store_elem(y, r, yv);
        }
    }
}

template <int N, typename T>
hipError_t launch_typed(const StepArgs &a, hipStream_t stream)
{
    const int64_t rows = a.batch * a.dim;
    const int64_t threads = rows * (N / 4);
    const int64_t blocks = (threads + kBlock - 1) / kBlock;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((state_update_kernel<N, T>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, a.state, (const T *)a.u, (const T *)a.delta, a.A,
                       (const T *)a.Bm, (const T *)a.Cm, a.D_skip, (const T *)a.z, a.delta_bias,
                       a.delta_softplus, (T *)a.y, a.dim, rows);
    return hipGetLastError();
}

template <int N>
hipError_t launch_n(const StepArgs &a, hipStream_t stream)
{
    return a.dtype == 1 ? launch_typed<N, uint16_t>(a, stream) : launch_typed<N, float>(a, stream);
}

} // namespace

hipError_t launch_state_update(const StepArgs &a, hipStream_t stream)
{
    switch (a.N) {
    case 4: return launch_n<4>(a, stream);
    case 8: return launch_n<8>(a, stream);
    case 16: return launch_n<16>(a, stream);
    case 32: return launch_n<32>(a, stream);
    case 64: return launch_n<64>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace selscan
