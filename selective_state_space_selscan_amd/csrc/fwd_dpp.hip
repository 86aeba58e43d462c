// Forward with an in-wave parallel scan over time (SELSCAN_FORCE_PLAN=dpp;
// an ablation of the streaming kernel's layout).
//
// The recurrence h_t = A_bar_t h_{t-1} + B_bar_t u_t composes affine maps
// h -> a h + b, an associative operation: applying (a1, b1) and then (a2, b2)
// gives (a2 a1, a2 b1 + b2) (selection-mechanism article, discosf.com §3.1;
// the parallel scan of the Mamba tutorial, pwwt.cn §3.2).  Here the 64 lanes
// of a wavefront hold 64 consecutive timesteps (a tile) of one channel, and
// each state's pairs are scanned across the lanes with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16, then the broadcasts of lane 15
// into rows 1 and 3 and of lane 31 into rows 2 and 3, which complete an
// inclusive scan of the 64 lanes (lanes without a source keep the identity).
// The state entering the tile (the previous tile's last lane, read into
// scalar registers) is then applied to every lane's inclusive pair:
// h_t = A_incl_t h_in + B_incl_t, and y_t is read out per lane.
//
// For structured A (A[d, n] = (n+1) A[d, 0]) the decay of a lane window is
// W^(n+1) with W the window's product of r = exp(Delta A[d, 0]), so the
// window products are scanned once per tile (six DPP rounds of a multiply)
// and each state takes its round factors as running powers; other A scans
// the decays of every state.
//
// Cost against the streaming kernel's sequential walk (4 operations per
// (t, n)): the scan's six rounds take a power step, a DPP move and an FMA per
// state each, about 25 operations per (t, n) with the carry and the readout;
// and the per-step inputs of a lane are one element of a different row
// (no coalescing across the wave).  One wave runs one channel, so a shape
// with few channels (batch * dim below 8192) also splits the sequence into
// parts, whose entry states come from the streaming forward's summary and
// carry passes.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace {

using stream::kLanes;

constexpr int kDppTile = kLanes;          // timesteps per tile (one per lane)
constexpr int64_t kDppTargetWaves = 8192; // waves the plan aims at (8 per SIMD)
constexpr int kRowShr = 0x110;            // DPP row_shr:k is kRowShr + k
constexpr int kRowBcast15 = 0x142;        // lane 15 of a row into the next row
constexpr int kRowBcast31 = 0x143;        // lane 31 into rows 2 and 3

// The value of an earlier lane moved by one scan round (j = 0..5), or
// `identity` on lanes without a source in that round.
template <int J>
__device__ __forceinline__ float from_earlier(float v, float identity)
{
    constexpr int ctrl = J < 4 ? kRowShr + (1 << J) : (J == 4 ? kRowBcast15 : kRowBcast31);
    constexpr int row_mask = J < 4 ? 0xf : (J == 4 ? 0xa : 0xc);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         __builtin_bit_cast(int, identity),
                                         __builtin_bit_cast(int, v), ctrl, row_mask, 0xf, false));
}

// One scan round of the pairs (a, b): the lane's pair follows the earlier
// window's: (a a_prev, a b_prev + b).
template <int J>
__device__ __forceinline__ void scan_round(float &a, float &b)
{
    const float ap = from_earlier<J>(a, 1.0f);
    const float bp = from_earlier<J>(b, 0.0f);
    b = fmaf(a, bp, b);
    a *= ap;
}

// The N values of row `row` of B or C (each lane its own row), as floats.
template <int N>
__device__ __forceinline__ void lane_row(const float *p, int64_t row, float (&v)[N])
{
    const float4 *q = reinterpret_cast<const float4 *>(p + row * N);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const float4 x = q[k];
        v[4 * k] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
    }
}
template <int N>
__device__ __forceinline__ void lane_row(const uint16_t *p, int64_t row, float (&v)[N])
{
    const uint2 *q = reinterpret_cast<const uint2 *>(p + row * N);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const uint2 x = q[k];
        v[4 * k] = __uint_as_float(x.x << 16);
        v[4 * k + 1] = __uint_as_float(x.x & 0xffff0000u);
        v[4 * k + 2] = __uint_as_float(x.y << 16);
        v[4 * k + 3] = __uint_as_float(x.y & 0xffff0000u);
    }
}

template <int N, bool POW, typename TIO>
__device__ __forceinline__ void dpp_part(const TIO *u, const TIO *delta, const TIO *z, TIO *y,
                                         const TIO *Bm, const TIO *Cm, int64_t b, int64_t d,
                                         int64_t L, int64_t dim, int64_t l0, int64_t l1,
                                         const float (&A2)[N], float A2_0, float bias, float Dd,
                                         int softplus_on, float (&hin)[N])
{
    const int lane = threadIdx.x & (kLanes - 1);
    for (int64_t t0 = l0; t0 < l1; t0 += kDppTile) {
        const int rows = (int)(l1 - t0 < kDppTile ? l1 - t0 : kDppTile);
        const bool valid = lane < rows;
        const int64_t row = b * L + t0 + (valid ? lane : 0);   // lanes past the end reuse step t0
        const int64_t e = row * dim + d;
        const float ut = load_elem(u, e);
        const float xr = load_elem(delta, e) + bias;
        const float sp = softplus(xr);
        const float dt = valid ? (softplus_on ? sp : xr) : 0.0f;   // padding: the identity
        const float du = dt * ut;
        float Bv[N], Cv[N];
        lane_row<N>(Bm, row, Bv);   // per lane: the row of its own step
        lane_row<N>(Cm, row, Cv);
        float yv = Dd * ut;
        const int last = rows - 1;
        if constexpr (POW) {
            // window products of r before each round, and the inclusive one
            float W[7];
            W[0] = exp2_decay(dt * A2_0, tag<TIO>());
            W[1] = W[0] * from_earlier<0>(W[0], 1.0f);
            W[2] = W[1] * from_earlier<1>(W[1], 1.0f);
            W[3] = W[2] * from_earlier<2>(W[2], 1.0f);
            W[4] = W[3] * from_earlier<3>(W[3], 1.0f);
            W[5] = W[4] * from_earlier<4>(W[4], 1.0f);
            W[6] = W[5] * from_earlier<5>(W[5], 1.0f);
            float P[7];
#pragma unroll
            for (int j = 0; j < 7; ++j)
                P[j] = 1.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
#pragma unroll
                for (int j = 0; j < 7; ++j)
                    P[j] *= W[j];   // W_j^(n+1)
                float bb = du * Bv[n];
                bb = fmaf(P[0], from_earlier<0>(bb, 0.0f), bb);
                bb = fmaf(P[1], from_earlier<1>(bb, 0.0f), bb);
                bb = fmaf(P[2], from_earlier<2>(bb, 0.0f), bb);
                bb = fmaf(P[3], from_earlier<3>(bb, 0.0f), bb);
                bb = fmaf(P[4], from_earlier<4>(bb, 0.0f), bb);
                bb = fmaf(P[5], from_earlier<5>(bb, 0.0f), bb);
                const float h = fmaf(P[6], hin[n], bb);
                yv = fmaf(Cv[n], h, yv);
                hin[n] = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h), last));
            }
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) {
                float a = exp2_decay(dt * A2[n], tag<TIO>());
                float bb = du * Bv[n];
                scan_round<0>(a, bb);
                scan_round<1>(a, bb);
                scan_round<2>(a, bb);
                scan_round<3>(a, bb);
                scan_round<4>(a, bb);
                scan_round<5>(a, bb);
                const float h = fmaf(a, hin[n], bb);
                yv = fmaf(Cv[n], h, yv);
                hin[n] = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h), last));
            }
        }
        if (z)
            yv *= silu(load_elem(z, e));
        if (valid)
            store_elem(y, e, yv);
    }
}

// One wave per (batch row, channel, sequence part); consecutive waves take
// consecutive channels, so the strided per-lane loads of neighbouring waves
// share cache lines.
template <int N, typename TIO>
__global__ __launch_bounds__(kLanes * 4) void fwd_dpp_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    TIO *__restrict__ y, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ h0,
    float *__restrict__ h_last, const float *__restrict__ entry, int64_t L, int64_t dim,
    int64_t chans, int parts, int64_t part_len)
{
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= chans * parts)
        return;
    const int part = (int)(w / chans);
    const int64_t bd = w % chans;
    const int64_t b = bd / dim, d = bd % dim;
    const int64_t l0 = (int64_t)part * part_len;
    const int64_t l1 = l0 + part_len < L ? l0 + part_len : L;
    const float A0 = A[d * N];
    float A2[N];
    bool structured = true;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    const float bias = delta_bias ? delta_bias[d] : 0.0f;
    const float Dd = D_skip ? D_skip[d] : 0.0f;
    // the state entering the part: h0 for the first, else the carry's entry
    // state (layout (channel groups, parts, N, 64))
    float hin[N];
    const int64_t gpr = (dim + kLanes - 1) / kLanes;
    const int64_t grp = b * gpr + d / kLanes;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        if (part == 0)
            hin[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0f;
        else
            hin[n] = entry[((grp * parts + part) * N + n) * kLanes + d % kLanes];
    }
    if (structured)
        dpp_part<N, true>(u, delta, z, y, Bm, Cm, b, d, L, dim, l0, l1, A2, A0 * kLog2e, bias,
                          Dd, delta_softplus, hin);
    else
        dpp_part<N, false>(u, delta, z, y, Bm, Cm, b, d, L, dim, l0, l1, A2, A0 * kLog2e, bias,
                           Dd, delta_softplus, hin);
    if (h_last && part == parts - 1 && (threadIdx.x & (kLanes - 1)) == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h_last[(b * dim + d) * N + n] = hin[n];
    }
}

// Parts so that batch * dim * parts reaches kDppTargetWaves, whole tiles each
// (at most the default forward's part count, whose workspace this shares).
StreamPlan dpp_plan(int64_t batch, int64_t L, int64_t dim)
{
    const StreamPlan def = default_fwd_plan(batch, L, dim);
    const int64_t chans = batch * dim;
    int64_t parts = (kDppTargetWaves + chans - 1) / chans;
    if (parts > def.parts)
        parts = def.parts;
    if (parts < 1)
        parts = 1;
    StreamPlan p;
    p.groups = def.groups;
    p.part_len = (L + parts - 1) / parts;
    p.part_len = (p.part_len + kDppTile - 1) / kDppTile * kDppTile;
    p.parts = (int)((L + p.part_len - 1) / p.part_len);
    return p;
}

template <int N, typename TIO>
hipError_t launch_t(const FwdArgs &a, const StreamPlan &p, float *entry, hipStream_t s)
{
    const int64_t chans = a.batch * a.dim;
    const int64_t blocks = (chans * p.parts + 3) / 4;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_dpp_kernel<N, TIO>), dim3((unsigned)blocks), dim3(kLanes * 4), 0, s,
                       (const TIO *)a.u, (const TIO *)a.delta, (const TIO *)a.z, (TIO *)a.y, a.A,
                       (const TIO *)a.Bm, (const TIO *)a.Cm, a.D_skip, a.delta_bias,
                       a.delta_softplus, a.h0, a.h_last, (const float *)entry, a.L, a.dim, chans,
                       p.parts, p.part_len);
    return hipGetLastError();
}

} // namespace

size_t fwd_dpp_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    const StreamPlan p = dpp_plan(batch, L, dim);
    if (p.parts <= 1)
        return 0;
    const size_t summ = (size_t)p.groups * (p.parts - 1) * (N + 1) * kLanes * 4;
    const size_t entry = (size_t)p.groups * p.parts * N * kLanes * 4;
    return 256 + ((summ + 255) & ~(size_t)255) + ((entry + 255) & ~(size_t)255) +
           carry_scratch_bytes(p.groups, p.parts, N);
}

hipError_t launch_fwd_dpp(const FwdArgs &a, hipStream_t stream)
{
    const StreamPlan p = dpp_plan(a.batch, a.L, a.dim);
    float *entry = nullptr;
    if (p.parts > 1) {
        // the parts' entry states: the streaming forward's summary pass over
        // this plan's parts, then its carry of h0 through the summaries
        float *summ = stream::summary_buffer(a.workspace);
        entry = stream::entry_buffer(a.workspace, p, a.N);
        hipError_t err = launch_fwd_summaries(a, p, summ, stream);
        if (err == hipSuccess)
            err = launch_fwd_carry(summ, a.h0, a.A, entry, a.batch, a.dim, a.N, p.parts, 0,
                                   stream::carry_scratch(a.workspace, p, a.N), stream);
        if (err != hipSuccess)
            return err;
    }
#define SELSCAN_DPP_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return a.dtype == 1 ? launch_t<NN, uint16_t>(a, p, entry, stream)                         \
                            : launch_t<NN, float>(a, p, entry, stream);
    switch (a.N) {
    SELSCAN_DPP_CASE(4)
    SELSCAN_DPP_CASE(8)
    SELSCAN_DPP_CASE(16)
    SELSCAN_DPP_CASE(32)
    SELSCAN_DPP_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_DPP_CASE
}

} // namespace selscan
