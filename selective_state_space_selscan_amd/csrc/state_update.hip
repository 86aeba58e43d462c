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
// of a wave covers 1 KB of contiguous memory.  Each lane updates its 4 states
// in two rows (the block's two runs of consecutive rows), forms its part of
// C.h, and the row's lanes sum the parts with xor-shuffles.
// The per-row scalars (Delta, u, z) are recomputed by every lane of the row,
// which costs nothing measurable in a memory-bound step.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace {

constexpr int kBlock = 256;
// Rows per lane, loads of all of them issued first: 2 puts two state loads
// in flight per lane.  Measured on batch 256, D 5120, N 16 (cold step, the
// state from HBM): 35.4 us at 2 rows per lane, 37.8 at 1, 38.1 at 4; one
// lane per row (all 16 states in a lane, its loads 64 B apart across the
// wave) 44.7; a persistent grid loading the next chunk while updating the
// current one 39-45; non-temporal state loads and stores 36.5.
constexpr int kStateRowsPerLane = 2;

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

template <int N, typename T, int K>
__global__ __launch_bounds__(kBlock) void state_update_kernel(
    float *__restrict__ state, const T *__restrict__ u, const T *__restrict__ delta,
    const float *__restrict__ A, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ D_skip, const T *__restrict__ z,
    const float *__restrict__ delta_bias, int delta_softplus, T *__restrict__ y, uint32_t dim,
    double inv_dim, uint32_t rows)
{
    static_assert(N % 4 == 0 && kBlock % (N / 4) == 0, "N/4 lanes per row");
    constexpr uint32_t R = N / 4;                       // lanes per (b, d) row
    constexpr uint32_t kRowsPerSlot = kBlock / R;       // rows one slot of the block covers
    // K slots per lane: the block covers K * kRowsPerSlot consecutive rows, slot
    // k the k-th run of kRowsPerSlot.  All K rows' loads are issued before any
    // row is computed and stored, so each lane has K state loads in flight.
    // Indices are 32-bit (rows * N < 2^31 is checked on the host); b = row /
    // dim comes from a double-precision reciprocal, exact after one
    // correction step for row < 2^31.
    const uint32_t q = threadIdx.x % R;                 // this lane's float4 of a row
    const uint32_t row0 = blockIdx.x * (K * kRowsPerSlot) + threadIdx.x / R;
    float4 h4[K], a4[K];
    float Bv[K][4], Cv[K][4], ut[K], xr[K], zt[K], Dd[K];
    uint32_t r[K];
    bool valid[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t row = row0 + k * kRowsPerSlot;
        valid[k] = row < rows;
        r[k] = valid[k] ? row : rows - 1;          // tail lanes compute on a valid row
        uint32_t b = (uint32_t)((double)r[k] * inv_dim);
        int64_t dd = (int64_t)r[k] - (int64_t)b * dim;
        if (dd < 0) { --b; dd += dim; }
        if (dd >= (int64_t)dim) { ++b; dd -= dim; }
        const uint32_t d = (uint32_t)dd;
        h4[k] = *(reinterpret_cast<const float4 *>(state + r[k] * N) + q);
        a4[k] = *reinterpret_cast<const float4 *>(A + d * N + 4 * q);
        load4<T>(Bm + b * N + 4 * q, Bv[k]);
        load4<T>(Cm + b * N + 4 * q, Cv[k]);
        ut[k] = load_elem(u, r[k]);
        xr[k] = load_elem(delta, r[k]) + (delta_bias ? delta_bias[d] : 0.0f);
        zt[k] = z ? load_elem(z, r[k]) : 0.0f;
        Dd[k] = D_skip ? D_skip[d] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float dt = delta_softplus ? softplus(xr[k]) : xr[k];
        const float du = dt * ut[k];
        const float dA = dt * kLog2e;
        float h[4] = {h4[k].x, h4[k].y, h4[k].z, h4[k].w};
        const float a[4] = {a4[k].x, a4[k].y, a4[k].z, a4[k].w};
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
                float yv = fmaf(Dd[k], ut[k], acc);
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
    constexpr int64_t rows_per_block = kStateRowsPerLane * (kBlock / (N / 4));
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((state_update_kernel<N, T, kStateRowsPerLane>), dim3((unsigned)blocks),
                       dim3(kBlock), 0,
                       stream, a.state, (const T *)a.u, (const T *)a.delta, a.A,
                       (const T *)a.Bm, (const T *)a.Cm, a.D_skip, (const T *)a.z, a.delta_bias,
                       a.delta_softplus, (T *)a.y, (uint32_t)a.dim, 1.0 / (double)a.dim,
                       (uint32_t)rows);
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
