// Chunked selective-scan forward for gfx950 (an ablation plan, SELSCAN_FORCE_PLAN=chunked;
// measured slower than the streaming plan, which is the default).
//
// What it computes is the S6 recurrence of the Mamba tutorial (pwwt.cn)
// §3.1-§3.2 and §4.2: Delta_t = softplus(Delta_raw + bias), A_bar = exp(Delta_t A)
// with diagonal A, h_t = A_bar_t h_{t-1} + Delta_t B_t u_t, y_t = C_t.h_t + D u_t,
// times SiLU(z_t).  The sequence axis is split and recombined with the
// associative operator of the selection-mechanism article (discosf.com) §3.1:
// (a, b) o (c, d) = (a c, a d + b), the later element on the left.
//
// Work decomposition (one workgroup = W wavefronts x 64 lanes):
//   * lane    = one channel d of a 64-channel group (fixed batch row b), so the
//               u/Delta/z/y accesses of a wave are one contiguous 128 B (bf16)
//               row per timestep, and B_t, C_t are the same for every lane:
//               they are read as scalar (SGPR) operands.
//   * wave w  = segment w of T timesteps of the current chunk (W*T timesteps).
//   * the workgroup walks its L range chunk by chunk; the state entering a
//     chunk (the carry) lives in LDS, never in HBM.
// Per chunk and per state index n:
//   1. each wave runs its segment's recurrence from zero (the local chain),
//      giving the segment aggregate (P, x): P = prod A_bar = exp2(A2[n] sum Delta),
//      x = local end state;
//   2. aggregates go to LDS; after one barrier each wave folds the carry and
//      the aggregates of the segments before it into its entry state;
//   3. each wave re-runs its segment from that entry state and accumulates
//      C_t[n] h_t into y_t (the fix-up chain); the last wave's end state is the
//      next chunk's carry.
// The per-(t,n) factors A_bar and Delta B u are computed once and kept in VGPRs
// between the two chains.  The hidden state is never written to HBM (Gu & Dao
// deep-reading report §2.4); only y and, if asked, h_L are.
//
// Structured A: when every A[d, n] equals (n+1) A[d, 0] exactly (the S4D-real
// initialisation A = -exp(log(1..N)) of the tutorial's §4.2 listing), then
// exp(Delta A[d,n]) = r^(n+1) with r = exp(Delta A[d,0]).  A wave whose 64 channels
// all have this structure computes A_bar by one multiply per (t, n) instead of
// a multiply and an exp2.  Any other A takes the exp2 path; both are exact
// readings of exp(Delta A) up to rounding.
//
// Long sequences: the L axis may also be split into P parts handled by
// different workgroups.  A summary pass (SUMMARY = true) computes, for every
// part but the last, the part's aggregate (sum Delta, end state from zero) into
// the workspace; the main pass folds the aggregates of the parts before its own
// into its initial carry.
#include "buffer_io.hpp"
#include "device_math.hpp"
#include "kernels.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace selscan {
namespace {

constexpr int kLanes = 64;

// ----------------------------------------------------------------------------
// B and C (batch, L, N) -> fp32 (batch, N, Lpad), zero-padded past L, so that
// a wave reads the T values of one state index n as one contiguous scalar load.
// ----------------------------------------------------------------------------
template <typename TIO>
__global__ __launch_bounds__(256) void bc_transpose_kernel(
    const TIO *__restrict__ Bm, const TIO *__restrict__ Cm, float *__restrict__ BT,
    float *__restrict__ CT, int64_t L, int64_t Lpad, int N)
{
    const int64_t b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= Lpad)
        return;
    const bool valid = t < L;
    for (int n = 0; n < N; ++n) {
        const int64_t src = (b * L + t) * N + n;
        const int64_t dst = (b * N + n) * Lpad + t;
        BT[dst] = valid ? load_elem(Bm, src) : 0.0f;
        CT[dst] = valid ? load_elem(Cm, src) : 0.0f;
    }
}

// Phase A of one chunk for one wave: per-timestep quantities of the wave's
// T-step segment.  All loads are issued before any arithmetic so that one
// memory round trip covers the whole segment.
template <int T, bool SUMMARY, bool SOFTPLUS, typename TIO>
__device__ __forceinline__ void phase_a(const TIO *u, const TIO *delta, const TIO *z,
                                        int64_t seg_elem, int64_t seg_bytes, int voff,
                                        int row_bytes, int rows, float bias, float Dd,
                                        bool pow_path, float A2_0, float (&du)[T],
                                        float (&rr)[T], float (&yv)[T], float (&gt)[T],
                                        float &sdelta)
{
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + seg_elem, seg_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + seg_elem, seg_bytes);
    float uv[T], xv[T], zv[T];
#pragma unroll
    for (int i = 0; i < T; ++i)
        xv[i] = buf_load(rd, voff, i * row_bytes, delta);
#pragma unroll
    for (int i = 0; i < T; ++i)
        uv[i] = buf_load(ru, voff, i * row_bytes, u);
    const bool gated = !SUMMARY && z != nullptr;
    if (gated) {
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + seg_elem, seg_bytes);
#pragma unroll
        for (int i = 0; i < T; ++i)
            zv[i] = buf_load(rz, voff, i * row_bytes, z);
    }
    sdelta = 0.0f;
#pragma unroll
    for (int i = 0; i < T; ++i) {
        const float x = xv[i] + bias;
        float dt = SOFTPLUS ? softplus(x) : x;
        dt = i < rows ? dt : 0.0f;   // padding steps are the identity (1, 0)
        du[i] = dt * uv[i];
        rr[i] = pow_path ? exp2_decay(dt * A2_0, (const TIO *)nullptr) : dt * kLog2e;
        sdelta += dt;
        if (!SUMMARY)
            yv[i] = Dd * uv[i];
    }
    if (!SUMMARY) {
#pragma unroll
        for (int i = 0; i < T; ++i)
            gt[i] = gated ? silu(zv[i]) : 1.0f;
    }
}

template <int N, int T, int W, bool SUMMARY, typename TIO>
__global__ __launch_bounds__(kLanes * W) void fwd_chunked_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    TIO *__restrict__ y, const float *__restrict__ A, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ h0,
    float *__restrict__ h_last, const float *__restrict__ BT, const float *__restrict__ CT,
    float *__restrict__ summ, int64_t L, int64_t dim, int64_t Lpad, int64_t part_len)
{
    constexpr int CH = W * T;   // timesteps per chunk
    constexpr int ES = (int)sizeof(TIO);
    static_assert(W % 4 == 0, "the fold reads aggregates four at a time");
    const int lane = threadIdx.x & (kLanes - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int64_t groups_per_row = (dim + kLanes - 1) / kLanes;
    const int64_t grp = blockIdx.x;
    const int64_t b = grp / groups_per_row;
    const int64_t d0 = (grp % groups_per_row) * kLanes;
    const bool active = d0 + lane < dim;
    const int64_t d = active ? d0 + lane : dim - 1;
    const int part = blockIdx.y;
    const int n_parts_total = SUMMARY ? gridDim.y + 1 : gridDim.y;
    const int64_t l_begin = (int64_t)part * part_len;
    const int64_t l_end = (l_begin + part_len < L) ? l_begin + part_len : L;
    const int voff = lane * ES;
    const int row_bytes = (int)(dim * ES);

    // Per-channel constants.
    const float A0 = A[d * N];
    bool structured = true;
#pragma unroll
    for (int n = 1; n < N; ++n)
        structured = structured && (A[d * N + n] == (float)(n + 1) * A0);
    // One path per wave: the power chain only if all 64 lanes qualify.
    const bool pow_path = __all(structured);
    const float A2_0 = A0 * kLog2e;
    const float Dd = (D_skip && !SUMMARY) ? D_skip[d] : 0.0f;
    const float bias = delta_bias ? delta_bias[d] : 0.0f;

    __shared__ float2 agg[2][W][kLanes];      // (P, x) per segment, by parity of n
    __shared__ float carry[2][N][kLanes];     // chunk carry, by parity of the chunk
    __shared__ float sum_part[W][kLanes];

    // Initial carry.  Summary pass: zero (every part's aggregate is taken from
    // a zero state).  Main pass: h0 (or 0), then the aggregates of the parts
    // before this one, folded in order.
    if (w == 0) {
        for (int n = 0; n < N; ++n) {
            float h = (h0 && !SUMMARY) ? h0[(b * dim + d) * N + n] : 0.0f;
            if (!SUMMARY) {
                const float a2n = A[d * N + n] * kLog2e;
                for (int q = 0; q < part; ++q) {
                    const float *s = summ + ((grp * (n_parts_total - 1) + q) * (N + 1)) * kLanes;
                    h = fmaf(hw_exp2(a2n * s[lane]), h, s[(n + 1) * kLanes + lane]);
                }
            }
            carry[0][n][lane] = h;
        }
    }
    float sdelta_total = 0.0f;
    __syncthreads();

    int c = 0;
    for (int64_t chunk0 = l_begin; chunk0 < l_end; chunk0 += CH, ++c) {
        const int64_t t0 = chunk0 + (int64_t)w * T;
        const int cp = c & 1;
        int64_t rows64 = l_end - t0;
        rows64 = rows64 < 0 ? 0 : (rows64 > T ? T : rows64);
        const int rows = (int)rows64;
        const int64_t seg_elem = (b * L + t0) * dim + d0;
        const int64_t seg_bytes = rows > 0 ? (rows64 * dim - d0) * ES : 0;

        // Phase A: per-timestep quantities of this wave's segment.
        float du[T], rr[T], yv[T], gt[T];
        float sdelta;
        if (delta_softplus)
            phase_a<T, SUMMARY, true>(u, delta, z, seg_elem, seg_bytes, voff, row_bytes, rows,
                                      bias, Dd, pow_path, A2_0, du, rr, yv, gt, sdelta);
        else
            phase_a<T, SUMMARY, false>(u, delta, z, seg_elem, seg_bytes, voff, row_bytes, rows,
                                       bias, Dd, pow_path, A2_0, du, rr, yv, gt, sdelta);
        sdelta_total += sdelta;

        // Phase B: one pass per state index n.
        float pw[T], in[T];
#pragma unroll
        for (int i = 0; i < T; ++i)
            pw[i] = 1.0f;
        const float Rseg = pow_path ? hw_exp2(sdelta * A2_0) : 0.0f;
        float Pseg = 1.0f;
        const const_f32 *bbase = as_const(BT) + (b * N * Lpad + t0);
        const const_f32 *cbase = as_const(CT) + (b * N * Lpad + t0);
#pragma unroll 1
        for (int n = 0; n < N; ++n) {
            // B and C columns of this n: scalar loads; C is consumed only
            // after the local chain and the barrier, which hide its latency.
            float bs[T], cs[T];
#pragma unroll
            for (int i = 0; i < T; ++i)
                bs[i] = bbase[n * Lpad + i];
#pragma unroll
            for (int i = 0; i < T; ++i)
                cs[i] = SUMMARY ? 0.0f : cbase[n * Lpad + i];
            if (pow_path) {
#pragma unroll
                for (int i = 0; i < T; ++i)
                    pw[i] *= rr[i];
                Pseg *= Rseg;
            } else {
                const float an = A[d * N + n];
#pragma unroll
                for (int i = 0; i < T; ++i)
                    pw[i] = exp2_decay(rr[i] * an, (const TIO *)nullptr);
                Pseg = hw_exp2(sdelta * kLog2e * an);
            }
            float x = 0.0f;
#pragma unroll
            for (int i = 0; i < T; ++i) {
                in[i] = du[i] * bs[i];
                x = fmaf(pw[i], x, in[i]);
            }
            const int np = n & 1;
            agg[np][w][lane] = make_float2(Pseg, x);
            __syncthreads();
            float h = carry[cp][n][lane];
            const int nfold = SUMMARY ? (w == W - 1 ? W : 0) : w;
            for (int k0 = 0; k0 < nfold; k0 += 4) {
                const float2 a0 = agg[np][k0][lane];
                const float2 a1 = agg[np][k0 + 1][lane];
                const float2 a2 = agg[np][k0 + 2][lane];
                const float2 a3 = agg[np][k0 + 3][lane];
                h = fmaf(a0.x, h, a0.y);
                if (k0 + 1 < nfold)
                    h = fmaf(a1.x, h, a1.y);
                if (k0 + 2 < nfold)
                    h = fmaf(a2.x, h, a2.y);
                if (k0 + 3 < nfold)
                    h = fmaf(a3.x, h, a3.y);
            }
            if (!SUMMARY) {
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    h = fmaf(pw[i], h, in[i]);
                    yv[i] = fmaf(cs[i], h, yv[i]);
                }
            }
            if (w == W - 1)
                carry[cp ^ 1][n][lane] = h;
        }

        // Phase C: gate and store (lanes past dim store nothing; rows past the
        // end of the range fall outside the descriptor and are dropped).
        if (!SUMMARY && active) {
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + seg_elem, seg_bytes);
#pragma unroll
            for (int i = 0; i < T; ++i)
                buf_store(ry, voff, i * row_bytes, yv[i] * gt[i], y);
        }
    }

    // The carry after the last chunk is this part's end state.
    if (SUMMARY)
        sum_part[w][lane] = sdelta_total;
    __syncthreads();
    const int cf = c & 1;
    if (SUMMARY) {
        if (w == 0) {
            float s = 0.0f;
            for (int k = 0; k < W; ++k)
                s += sum_part[k][lane];
            float *o = summ + ((grp * (n_parts_total - 1) + part) * (N + 1)) * kLanes;
            o[lane] = s;
            for (int n = 0; n < N; ++n)
                o[(n + 1) * kLanes + lane] = carry[cf][n][lane];
        }
    } else if (h_last && active && w == 0 && part == (int)gridDim.y - 1) {
        for (int n = 0; n < N; ++n)
            h_last[(b * dim + d) * N + n] = carry[cf][n][lane];
    }
}

struct Plan {
    int W, T;
    int64_t chunk, Lpad, part_len;
    int parts;
    int64_t groups;
};

constexpr int kT = 16;

// SELSCAN_CHUNKED_PLAN="W,P" overrides the waves per workgroup (4, 8 or 16)
// and the number of sequence parts (tuning knob; P is capped as below).
bool plan_override(int *W, int64_t *P)
{
    const char *e = getenv("SELSCAN_CHUNKED_PLAN");
    if (!e)
        return false;
    int w = 0;
    long long p = 0;
    if (sscanf(e, "%d,%lld", &w, &p) != 2 || (w != 4 && w != 8 && w != 16) || p < 1)
        return false;
    *W = w;
    *P = p;
    return true;
}

Plan make_plan(int64_t batch, int64_t L, int64_t dim)
{
    Plan p;
    p.T = kT;
    p.groups = batch * ((dim + kLanes - 1) / kLanes);
    p.W = p.groups >= 1024 ? 4 : (p.groups >= 384 ? 8 : 16);
    int oW = 0;
    int64_t oP = 0;
    const bool over = plan_override(&oW, &oP);
    if (over)
        p.W = oW;
    p.chunk = (int64_t)p.W * p.T;
    const int64_t chunks = (L + p.chunk - 1) / p.chunk;
    // Split L across workgroups only when the groups alone leave the chip
    // idle; every part keeps at least 4 chunks.
    const int64_t target_waves = 4096;
    int64_t parts = over ? oP : target_waves / (p.groups * p.W);
    if (!over && parts > chunks / 4)
        parts = chunks / 4;
    if (parts > chunks)
        parts = chunks;
    if (parts < 1)
        parts = 1;
    if (parts > 4096)
        parts = 4096;
    const int64_t chunks_per_part = (chunks + parts - 1) / parts;
    p.part_len = chunks_per_part * p.chunk;
    p.parts = (int)((L + p.part_len - 1) / p.part_len);
    p.Lpad = (int64_t)p.parts * p.part_len;
    return p;
}

size_t bc_bytes(const Plan &p, int64_t batch, int64_t N) { return 2 * (size_t)batch * N * p.Lpad * 4; }

size_t summ_bytes(const Plan &p, int64_t N)
{
    return p.parts > 1 ? (size_t)p.groups * (p.parts - 1) * (N + 1) * kLanes * 4 : 0;
}

template <int N, int W, typename TIO>
hipError_t launch_wn(const FwdArgs &a, const Plan &p, float *BT, float *CT, float *summ,
                     hipStream_t s)
{
    if (p.parts > 1) {
        hipLaunchKernelGGL((fwd_chunked_kernel<N, kT, W, true, TIO>),
                           dim3((unsigned)p.groups, (unsigned)(p.parts - 1)), dim3(kLanes * W), 0,
                           s, (const TIO *)a.u, (const TIO *)a.delta, (const TIO *)nullptr,
                           (TIO *)nullptr, a.A, (const float *)nullptr, a.delta_bias,
                           a.delta_softplus, a.h0, (float *)nullptr, BT, CT, summ, a.L, a.dim,
                           p.Lpad, p.part_len);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((fwd_chunked_kernel<N, kT, W, false, TIO>),
                       dim3((unsigned)p.groups, (unsigned)p.parts), dim3(kLanes * W), 0, s,
                       (const TIO *)a.u, (const TIO *)a.delta, (const TIO *)a.z, (TIO *)a.y, a.A,
                       a.D_skip, a.delta_bias, a.delta_softplus, a.h0, a.h_last, BT, CT, summ,
                       a.L, a.dim, p.Lpad, p.part_len);
    return hipGetLastError();
}

template <int N, typename TIO>
hipError_t launch_n(const FwdArgs &a, const Plan &p, float *BT, float *CT, float *summ,
                    hipStream_t s)
{
    hipLaunchKernelGGL((bc_transpose_kernel<TIO>),
                       dim3((unsigned)((p.Lpad + 255) / 256), (unsigned)a.batch), dim3(256), 0, s,
                       (const TIO *)a.Bm, (const TIO *)a.Cm, BT, CT, a.L, p.Lpad, (int)N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (p.W) {
    case 4: return launch_wn<N, 4, TIO>(a, p, BT, CT, summ, s);
    case 8: return launch_wn<N, 8, TIO>(a, p, BT, CT, summ, s);
    default: return launch_wn<N, 16, TIO>(a, p, BT, CT, summ, s);
    }
}

template <typename TIO>
hipError_t launch_t(const FwdArgs &a, const Plan &p, float *BT, float *CT, float *summ,
                    hipStream_t s)
{
    switch (a.N) {
    case 4: return launch_n<4, TIO>(a, p, BT, CT, summ, s);
    case 8: return launch_n<8, TIO>(a, p, BT, CT, summ, s);
    case 16: return launch_n<16, TIO>(a, p, BT, CT, summ, s);
    case 32: return launch_n<32, TIO>(a, p, BT, CT, summ, s);
    case 64: return launch_n<64, TIO>(a, p, BT, CT, summ, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

size_t fwd_chunked_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    const Plan p = make_plan(batch, L, dim);
    return bc_bytes(p, batch, N) + summ_bytes(p, N) + 256;
}

hipError_t launch_fwd_chunked(const FwdArgs &a, hipStream_t stream)
{
    const Plan p = make_plan(a.batch, a.L, a.dim);
    uintptr_t base = ((uintptr_t)a.workspace + 255) & ~(uintptr_t)255;
    float *BT = (float *)base;
    float *CT = BT + (size_t)a.batch * a.N * p.Lpad;
    float *summ = CT + (size_t)a.batch * a.N * p.Lpad;
    return a.dtype == 1 ? launch_t<uint16_t>(a, p, BT, CT, summ, stream)
                        : launch_t<float>(a, p, BT, CT, summ, stream);
}

} // namespace selscan
