// Decode step for gfx950: one t-step of the selective recurrence applied in
// place to a resident fp32 state (batch, dim, N).
//
// Decode keeps one fixed-size state per sample and does O(1) work per token
// (Mamba tutorial, pwwt.cn, §5.1 table and §6.3).  The paper walkthrough
// (m.lqnn.cn) §3.2 names this single-token state update.  The step is
// HBM-bound: each state entry is read once and written once, 8 bytes per
// (b, d, n), against 5 flops and one exp2.
//
// One lane owns one (b, d) row of N states (N*4 contiguous bytes, loaded as
// float4).  B and C of row b are wave-uniform.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace {

constexpr int kBlock = 256;

template <int N, typename T>
__global__ __launch_bounds__(kBlock) void state_update_kernel(
    float *__restrict__ state, const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D_skip, const T *__restrict__ z,
    const float *__restrict__ delta_bias, int delta_softplus, T *__restrict__ y, int64_t dim)
{
    static_assert(N % 4 == 0, "N must be a multiple of 4");
    const int64_t b = blockIdx.y;
    const int64_t d = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (d >= dim)
        return;
    const int64_t e = b * dim + d;
    float4 *row = reinterpret_cast<float4 *>(state + e * N);
    const T *Bt = Bm + b * N;
    const T *Ct = Cm + b * N;

    const float ut = load_elem(u, e);
    const float x = load_elem(delta, e) + (delta_bias ? delta_bias[d] : 0.0f);
    const float dt = delta_softplus ? softplus(x) : x;
    const float du = dt * ut;
    const float dA = dt * kLog2e;
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        float4 hv = row[q];
        float4 av = *reinterpret_cast<const float4 *>(A + d * N + 4 * q);
        float hs[4] = {hv.x, hv.y, hv.z, hv.w};
        float as[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = 4 * q + k;
            hs[k] = fmaf(hw_exp2(dA * as[k]), hs[k], du * load_elem(Bt, n));
            acc = fmaf(load_elem(Ct, n), hs[k], acc);
        }
        row[q] = make_float4(hs[0], hs[1], hs[2], hs[3]);
    }
    float yv = fmaf(D_skip ? D_skip[d] : 0.0f, ut, acc);
    if (z)
        yv *= silu(load_elem(z, e));
    store_elem(y, e, yv);
}

template <int N, typename T>
hipError_t launch_typed(const StepArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.dim + kBlock - 1) / kBlock), (unsigned)a.batch);
    hipLaunchKernelGGL((state_update_kernel<N, T>), grid, dim3(kBlock), 0, stream, a.state,
                       (const T *)a.u, (const T *)a.delta, a.A, (const T *)a.Bm,
                       (const T *)a.Cm, a.D_skip, (const T *)a.z, a.delta_bias,
                       a.delta_softplus, (T *)a.y, a.dim);
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
