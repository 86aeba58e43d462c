// Serial selective-scan forward for gfx950: one lane per (batch, channel),
// the whole sequence walked in-lane with the N-entry state in VGPRs.
//
// This is the plain recurrence of the Mamba tutorial (pwwt.cn) §4.2 fused
// into one kernel as §3.2 of the same page and the Gu & Dao report §2.4
// describe (discretise, scan and read out on chip, write only y).  Lanes run
// along the channel axis, so the u/Delta/z/y accesses of a wave are
// contiguous, and B_t, C_t (shared by all channels) are wave-uniform loads.
// It needs no workspace and handles every shape.  Its parallelism is only
// batch*dim lanes, so the chunked kernel takes over when that is too few.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace {

constexpr int kBlock = 256;

template <int N, typename T>
__global__ __launch_bounds__(kBlock) void fwd_serial_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm, const float *__restrict__ D_skip,
    const T *__restrict__ z, const float *__restrict__ delta_bias, int delta_softplus,
    const float *__restrict__ h0, T *__restrict__ y, float *__restrict__ h_last,
    int64_t L, int64_t dim)
{
    const int64_t b = blockIdx.y;
    const int64_t d_raw = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const bool active = d_raw < dim;
    const int64_t d = active ? d_raw : dim - 1;   // tail lanes compute on a valid channel, store nothing

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = A[d * N + n] * kLog2e;
        h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0f;
    }
    const float Dd = D_skip ? D_skip[d] : 0.0f;
    const float bias = delta_bias ? delta_bias[d] : 0.0f;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t e = (b * L + t) * dim + d;
        const T *Bt = Bm + (b * L + t) * N;
        const T *Ct = Cm + (b * L + t) * N;
        const float ut = load_elem(u, e);
        const float x = load_elem(delta, e) + bias;
        const float dt = delta_softplus ? softplus(x) : x;
        const float du = dt * ut;
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float a = hw_exp2(dt * A2[n]);
            h[n] = fmaf(a, h[n], du * load_elem(Bt, n));
            acc = fmaf(load_elem(Ct, n), h[n], acc);
        }
        float yv = fmaf(Dd, ut, acc);
        if (z)
            yv *= silu(load_elem(z, e));
        if (active)
            store_elem(y, e, yv);
    }
    if (h_last && active) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h_last[(b * dim + d) * N + n] = h[n];
    }
}

template <int N, typename T>
hipError_t launch_typed(const FwdArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.dim + kBlock - 1) / kBlock), (unsigned)a.batch);
    hipLaunchKernelGGL((fwd_serial_kernel<N, T>), grid, dim3(kBlock), 0, stream,
                       (const T *)a.u, (const T *)a.delta, a.A, (const T *)a.Bm,
                       (const T *)a.Cm, a.D_skip, (const T *)a.z, a.delta_bias,
                       a.delta_softplus, a.h0, (T *)a.y, a.h_last, a.L, a.dim);
    return hipGetLastError();
}

template <int N>
hipError_t launch_n(const FwdArgs &a, hipStream_t stream)
{
    return a.dtype == 1 ? launch_typed<N, uint16_t>(a, stream) : launch_typed<N, float>(a, stream);
}

} // namespace

hipError_t launch_fwd_serial(const FwdArgs &a, hipStream_t stream)
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
