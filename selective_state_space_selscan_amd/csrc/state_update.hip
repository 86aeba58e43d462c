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
// of a wave covers contiguous memory (1 KB for N = 16).  A workgroup covers
// kBlock / (N/4) consecutive channels d of kBatchesPerLane consecutive batch
// rows: each lane updates its 4 states of channel d in each of those rows,
// loading A[d], D[d] and the bias once for them, and issues all of their
// state loads before computing any (two in flight per lane).  Each lane forms
// its part of C.h and the row's lanes sum the parts with xor-shuffles.
// Measured on batch 256, D 5120, N 16 with the state coming from HBM: 31.8 us
// per step, against 34.7 us for the previous layout (two rows of different
// channels per lane, A read for each), 35.7 us with one batch row per lane
// and 31.9 us with four; 512-lane workgroups 32.3 us.  Earlier layouts, on
// the same shape: one lane per row (all 16 states in a lane, its loads 64 B
// apart across the wave) 44.7 us, a persistent grid loading the next rows
// while updating the current ones 39-45 us, non-temporal state stores no
// change.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace {

constexpr int kBlock = 256;
constexpr int kBatchesPerLane = 2;

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

// Indices are 32-bit: batch * dim * N < 2^31 is checked on the host.
template <int N, typename T, int KB>
__global__ __launch_bounds__(kBlock) void state_update_kernel(
    float *__restrict__ state, const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D_skip, const T *__restrict__ z,
    const float *__restrict__ delta_bias, int delta_softplus, T *__restrict__ y, uint32_t dim,
    uint32_t batch, uint32_t dblocks)
{
    static_assert(N % 4 == 0 && kBlock % (N / 4) == 0, "N/4 lanes per row");
    constexpr uint32_t R = N / 4;                // lanes per (b, d) row
    constexpr uint32_t kChans = kBlock / R;      // channels per workgroup
    const uint32_t q = threadIdx.x % R;          // this lane's float4 of a row
    const uint32_t b0 = (blockIdx.x / dblocks) * KB;
    const uint32_t d = (blockIdx.x % dblocks) * kChans + threadIdx.x / R;
    const bool dvalid = d < dim;
    const uint32_t dc = dvalid ? d : dim - 1;    // lanes past dim compute on a valid channel
    const float4 a4 = *reinterpret_cast<const float4 *>(A + dc * N + 4 * q);
    const float bias = delta_bias ? delta_bias[dc] : 0.0f;
    const float Dd = D_skip ? D_skip[dc] : 0.0f;
    float4 h4[KB];
    float Bv[KB][4], Cv[KB][4], ut[KB], xr[KB], zt[KB];
    uint32_t r[KB];
    bool valid[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const uint32_t b = b0 + k;
        valid[k] = dvalid && b < batch;
        const uint32_t bc = b < batch ? b : batch - 1;
        r[k] = bc * dim + dc;
        h4[k] = *(reinterpret_cast<const float4 *>(state + r[k] * N) + q);
        load4<T>(Bm + bc * N + 4 * q, Bv[k]);
        load4<T>(Cm + bc * N + 4 * q, Cv[k]);
        ut[k] = load_elem(u, r[k]);
        xr[k] = load_elem(delta, r[k]) + bias;
        zt[k] = z ? load_elem(z, r[k]) : 0.0f;
    }
    const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const float dt = delta_softplus ? softplus(xr[k]) : xr[k];
        const float du = dt * ut[k];
        const float dA = dt * kLog2e;
        float h[4] = {h4[k].x, h4[k].y, h4[k].z, h4[k].w};
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            h[m] = fmaf(exp2_decay(dA * a[m], (const T *)nullptr), h[m], du * Bv[k][m]);
            acc = fmaf(Cv[k][m], h[m], acc);
        }
        // sum C.h over the R lanes of the row (all lanes take part)
#pragma unroll
        for (uint32_t off = R / 2; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off, R);
        if (valid[k]) {
            *(reinterpret_cast<float4 *>(state + r[k] * N) + q) = make_float4(h[0], h[1], h[2], h[3]);
            if (q == 0) {
                float yv = fmaf(Dd, ut[k], acc);
                if (z)
                    yv *= silu(zt[k]);
                store_elem(y, r[k], yv);
            }
        }
    }
}

template <int N, typename T>
hipError_t launch_typed(const StepArgs &a, hipStream_t stream)
{
    const int64_t rows = a.batch * a.dim;
    if (rows * a.N >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;   // refused on the host before this point
    constexpr int64_t chans = kBlock / (N / 4);
    const int64_t dblocks = (a.dim + chans - 1) / chans;
    const int64_t blocks = (a.batch + kBatchesPerLane - 1) / kBatchesPerLane * dblocks;
    hipLaunchKernelGGL((state_update_kernel<N, T, kBatchesPerLane>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, stream, a.state, (const T *)a.u, (const T *)a.delta, a.A,
                       (const T *)a.Bm, (const T *)a.Cm, a.D_skip, (const T *)a.z, a.delta_bias,
                       a.delta_softplus, (T *)a.y, (uint32_t)a.dim, (uint32_t)a.batch,
                       (uint32_t)dblocks);
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
