// Backward of the selective scan for gfx950, with recomputation.
//
// Gradients of y = (C_t.h_t + D u_t) * SiLU(z_t), h_t = exp(Delta_t A) h_{t-1}
// + Delta_t B_t u_t (Euler B_bar, forward direction) for an upstream dy (and
// optionally dh_last).  The states are not stored by the forward: they are
// recomputed here (Gu & Dao deep-reading report §2.4; selection-mechanism
// article discosf.com §3.4).  The adjoint lambda_t = dL/dh_t runs backwards,
//   lambda_t = C_t dypre_t + A_bar_{t+1} lambda_{t+1},   dypre_t = dy_t SiLU(z_t),
// and every gradient is a per-step product of lambda_t, h_t and the inputs.
//
// Layout as in the streaming forward: lane = channel of a 64-channel group,
// wave = (group, sequence part), parts from the forward's plan.  Pipeline:
//   1. forward part summaries (the forward's summary pass);
//   2. adjoint part summaries, for the fold from the right: over a part
//      [s, e), the adjoint leaving it to the left is
//        g_{s-1} = sum_t (prod_{k=s..t} A_bar_k) C_t dypre_t
//                  + exp(A sum_part Delta) g_{e-1},
//      the same associative operator as the forward, in reverse;
//   3. checkpoints: each part walked forward from its entry state, storing
//      the state at the start of every TT-step chunk (fp32, in the workspace);
//   4. the main pass: each part walked backwards chunk by chunk; a chunk's
//      TT states are recomputed from its checkpoint into registers, then the
//      TT adjoint steps run.  Per-element gradients (du, ddelta, dz) are
//      stored directly; dB_t, dC_t (sums over channels) are reduced over the
//      wave's 64 lanes through LDS and written as one partial per channel
//      group; dA, dD, dbias (sums over batch and time) as one partial per wave;
//   5. a reduction of those partials.
// Every reduction has a fixed order, so the result is bitwise repeatable.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace {

using stream::kLanes;
using stream::RowRaw;
using stream::TT;
using stream::WaveCtx;
using stream::fetch_row;
using stream::row_val;

constexpr int kVar = stream::kVarExt;   // run-time softplus, forward direction, no variant
constexpr int kLdsStride = kLanes + 1;  // padded rows: conflict-free LDS transposes

// Per-wave setup shared by the backward kernels (the forward kernel's, with
// the same group/part decomposition).
struct WaveSetup {
    WaveCtx c;
    int64_t d, grp;
    int part, lane;
    bool active;
};

__device__ __forceinline__ bool setup_wave(WaveSetup &w, int64_t gw, int64_t groups,
                                           int waves_parts, int64_t L, int64_t dim,
                                           int64_t part_len, int elem_bytes)
{
    if (gw >= groups * waves_parts)
        return false;
    w.lane = threadIdx.x & (kLanes - 1);
    w.part = (int)(gw / groups);
    w.grp = gw % groups;
    const int64_t groups_per_row = (dim + kLanes - 1) / kLanes;
    WaveCtx &c = w.c;
    c.b = w.grp / groups_per_row;
    c.bL = c.b * L;
    c.d0 = (w.grp % groups_per_row) * kLanes;
    c.L = L;
    c.dim = dim;
    c.l_begin = (int64_t)w.part * part_len;
    c.l_end = c.l_begin + part_len < L ? c.l_begin + part_len : L;
    c.voff = w.lane * elem_bytes;
    c.row_bytes = (int)(dim * (int64_t)elem_bytes);
    w.active = c.d0 + w.lane < dim;
    w.d = w.active ? c.d0 + w.lane : dim - 1;
    c.voff_store = w.active ? c.voff : stream::kStoreOffsetOutOfRange;
    c.rev = 0;
    c.softplus = 0;
    c.invA0 = 0.0f;
    c.cb = 0.0f;
#pragma unroll
    for (int j = 0; j < stream::kMaxConv; ++j)
        c.cw[j] = 0.0f;
    return true;
}

// A2 = A log2(e) of this lane's channel; true when A[d,n] = (n+1) A[d,0] holds
// for every lane of the wave (the structured power chain applies).
template <int N>
__device__ __forceinline__ bool load_A(const float *A, int64_t d, float (&A2)[N], float &A2_0)
{
    const float A0 = A[d * N];
    bool structured = true;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    A2_0 = A0 * kLog2e;
    return __all(structured);
}

__device__ __forceinline__ float sigmoid(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

template <typename TIO>
__device__ __forceinline__ float raw_f(uint32_t v) { return raw_to_f32(v, tag<TIO>()); }

// Inputs of TT steps for the backward: u, Delta_raw, z, dy (raw bits).
struct BwdChunk {
    uint32_t u[TT], x[TT], z[TT], dy[TT];
};

// Loads the chunk at t0; chunks outside [l_begin, l_end) read nothing (zeros).
template <typename TIO>
__device__ __forceinline__ void load_bwd_chunk(BwdChunk &ch, const TIO *u, const TIO *delta,
                                               const TIO *z, const TIO *dy, const WaveCtx &c,
                                               int64_t t0, bool with_u)
{
    int64_t rows = c.l_end - t0;
    rows = rows < 0 ? 0 : (rows > TT ? TT : rows);
    if (t0 < c.l_begin)
        rows = 0;
    const int64_t elem = (c.bL + t0) * c.dim + c.d0;
    const int64_t bytes = rows > 0 ? (rows * c.dim - c.d0) * (int64_t)sizeof(TIO) : 0;
    const int64_t safe = rows > 0 ? elem : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(delta + safe, bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(dy + safe, bytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(with_u ? u + safe : nullptr, with_u ? bytes : 0);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z ? z + safe : nullptr, z ? bytes : 0);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        ch.x[i] = buf_load_raw(rx, c.voff, i * c.row_bytes, delta);
        ch.dy[i] = buf_load_raw(ry, c.voff, i * c.row_bytes, dy);
        ch.u[i] = buf_load_raw(ru, c.voff, i * c.row_bytes, u);
        ch.z[i] = buf_load_raw(rz, c.voff, i * c.row_bytes, z);
    }
}

// ---------------------------------------------------------------------------
// 2. adjoint part summaries (parts 1 .. P-1)
// ---------------------------------------------------------------------------
// Walks the part forwards: with Pr_t[n] = prod_{k=s..t} A_bar_k[n],
// v[n] = sum_t Pr_t[n] C_t[n] dypre_t.  For structured A, Pr_t[n] = P_t^(n+1)
// with P_t the running product of r_k = exp(Delta_k A[d,0]): a multiply and an
// FMA per (t, n), as in the forward summary.
template <int N, bool POW, typename TIO>
__device__ __forceinline__ void adjoint_summary_part(const TIO *delta, const TIO *z, const TIO *dy,
                                                     const TIO *Cm, const WaveCtx &c,
                                                     const float (&A2)[N], float (&v)[N],
                                                     float &sdelta)
{
    float Pn[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        Pn[n] = 1.0f;
    float P = 1.0f;
    BwdChunk A, B;
    int64_t t0 = c.l_begin;
    load_bwd_chunk(A, (const TIO *)nullptr, delta, z, dy, c, t0, false);
    for (;;) {
        load_bwd_chunk(B, (const TIO *)nullptr, delta, z, dy, c, t0 + TT, false);
        const int rows = (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            if (i >= rows)
                break;   // uniform: only the sequence end is partial
            RowRaw<N, TIO> crow;
            fetch_row(crow, Cm, c.bL + t0 + i);
            const float xr = raw_f<TIO>(A.x[i]) + c.bias;
            const float sp = softplus(xr);
            const float dt = c.softplus ? sp : xr;
            sdelta += dt;
            const float zt = raw_f<TIO>(A.z[i]);
            const float dypre = raw_f<TIO>(A.dy[i]) * (z ? silu(zt) : 1.0f);
            if (POW) {
                P *= hw_exp2(dt * c.A2_0);
                float pw = P * dypre;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    v[n] = fmaf(pw, row_val<N>(crow, n), v[n]);
                    pw *= P;
                }
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    Pn[n] *= hw_exp2(dt * A2[n]);
                    v[n] = fmaf(Pn[n] * dypre, row_val<N>(crow, n), v[n]);
                }
            }
        }
        t0 += TT;
        if (t0 >= c.l_end)
            break;
        A = B;
    }
}

template <int N, typename TIO>
__global__ __launch_bounds__(kLanes * 4) void bwd_adjoint_summary_kernel(
    const TIO *__restrict__ delta, const TIO *__restrict__ z, const TIO *__restrict__ dy,
    const float *__restrict__ A, const TIO *__restrict__ Cm, const float *__restrict__ delta_bias,
    int delta_softplus, float *__restrict__ asumm, int64_t L, int64_t dim, int64_t groups,
    int parts, int64_t part_len)
{
    WaveSetup w;
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (!setup_wave(w, gw, groups, parts - 1, L, dim, part_len, (int)sizeof(TIO)))
        return;
    // wave (grp, q) summarises part q + 1
    w.part += 1;
    WaveCtx &c = w.c;
    c.l_begin = (int64_t)w.part * part_len;
    c.l_end = c.l_begin + part_len < L ? c.l_begin + part_len : L;
    c.softplus = delta_softplus;
    float A2[N];
    const bool pow_path = load_A<N>(A, w.d, A2, c.A2_0);
    c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
    float v[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        v[n] = 0.0f;
    float sdelta = 0.0f;
    if (pow_path)
        adjoint_summary_part<N, true>(delta, z, dy, Cm, c, A2, v, sdelta);
    else
        adjoint_summary_part<N, false>(delta, z, dy, Cm, c, A2, v, sdelta);
    float *o = asumm + ((w.grp * (parts - 1) + (w.part - 1)) * (N + 1)) * kLanes + w.lane;
    o[0] = sdelta;
#pragma unroll
    for (int n = 0; n < N; ++n)
        o[(n + 1) * kLanes] = v[n];
}

// ---------------------------------------------------------------------------
// 3. checkpoints: the state entering every TT-step chunk
// ---------------------------------------------------------------------------
template <int N, bool POW, typename TIO>
__device__ __forceinline__ void checkpoint_part(const TIO *u, const TIO *delta, const TIO *Bm,
                                                const WaveCtx &c, const float (&A2)[N],
                                                float (&h)[N], float *ck)
{
    const float none[N] = {};
    float win[stream::kMaxConv - 1] = {};
    float sdelta = 0.0f;
    stream::Chunk A, B;
    int64_t t0 = c.l_begin;
    stream::load_chunk<false, kVar>(A, u, delta, (const TIO *)nullptr, c, t0);
    for (;;) {
        stream::load_chunk<false, kVar>(B, u, delta, (const TIO *)nullptr, c, t0 + TT);
        float *o = ck + (t0 / TT) * (N * kLanes);
#pragma unroll
        for (int n = 0; n < N; ++n)
            o[n * kLanes] = h[n];
        stream::run_any_chunk<N, true, false, true, POW, kVar>(A, Bm, Bm, (TIO *)nullptr, c, t0,
                                                               A2, none, h, sdelta, win);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
        A = B;
    }
}

template <int N, typename TIO>
__global__ __launch_bounds__(kLanes * 4) void bwd_checkpoint_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const float *__restrict__ A,
    const TIO *__restrict__ Bm, const float *__restrict__ delta_bias, int delta_softplus,
    const float *__restrict__ h0, const float *__restrict__ fsumm, float *__restrict__ ckpt,
    int64_t L, int64_t dim, int64_t groups, int parts, int64_t part_len, int64_t nck)
{
    WaveSetup w;
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (!setup_wave(w, gw, groups, parts, L, dim, part_len, (int)sizeof(TIO)))
        return;
    WaveCtx &c = w.c;
    c.softplus = delta_softplus;
    float A2[N];
    const bool pow_path = load_A<N>(A, w.d, A2, c.A2_0);
    c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
    c.Dd = 0.0f;
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        h[n] = h0 ? h0[(c.b * dim + w.d) * N + n] : 0.0f;
    stream::fold_summaries<N>(h, fsumm + (w.grp * (parts - 1)) * (N + 1) * kLanes + w.lane, 0,
                              w.part, 1, pow_path, A2, c.A2_0);
    float *ck = ckpt + w.grp * nck * (N * kLanes) + w.lane;
    if (pow_path)
        checkpoint_part<N, true>(u, delta, Bm, c, A2, h, ck);
    else
        checkpoint_part<N, false>(u, delta, Bm, c, A2, h, ck);
}

// ---------------------------------------------------------------------------
// 4. main backward pass
// ---------------------------------------------------------------------------
struct BwdOut {
    void *du, *ddelta, *dz;
    float *pB, *pC;     // (groups_per_row, batch, L, N) partial sums over 64 channels
    float *pA;          // (batch, parts, dim, N) partial sums over a part
    float *pD, *pbias;  // (batch, parts, dim)
    float *dh0;         // (batch, dim, N) or null
};

// TT steps: states recomputed from the chunk's checkpoint, then the adjoint
// steps from the last to the first.
template <int N, bool POW, typename TIO>
__device__ __forceinline__ void bwd_chunk(const BwdChunk &ch, const TIO *Bm, const TIO *Cm,
                                          const WaveCtx &c, int64_t t0, const float *ck,
                                          const float (&A2)[N], float (&g)[N], float (&dA)[N],
                                          float &dD, float &dbias, bool gated, const BwdOut &o,
                                          int64_t grp_in_row, int64_t batch, float *lds, int lane,
                                          bool active)
{
    const int rows = (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    // recompute h_t for the TT steps
    float hs[TT][N];
    {
        float h[N];
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = ck[n * kLanes];
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            RowRaw<N, TIO> brow;
            fetch_row(brow, Bm, c.bL + (i < rows ? t0 + i : t0));
            const float ut = raw_f<TIO>(ch.u[i]);
            const float xr = raw_f<TIO>(ch.x[i]) + c.bias;
            const float sp = softplus(xr);
            float dt = c.softplus ? sp : xr;
            dt = i < rows ? dt : 0.0f;
            const float du = dt * ut;
            const float r = POW ? hw_exp2(dt * c.A2_0) : 0.0f;
            float pw = 1.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float a = POW ? (pw *= r) : hw_exp2(dt * A2[n]);
                h[n] = fmaf(a, h[n], du * row_val<N>(brow, n));
                hs[i][n] = h[n];
            }
        }
    }
    // adjoint steps
    const int64_t elem = (c.bL + t0) * c.dim + c.d0;
    const int64_t bytes = (rows * c.dim - c.d0) * (int64_t)sizeof(TIO);
    const __amdgpu_buffer_rsrc_t rdu = make_rsrc((TIO *)o.du + elem, bytes);
    const __amdgpu_buffer_rsrc_t rdd = make_rsrc((TIO *)o.ddelta + elem, bytes);
    const __amdgpu_buffer_rsrc_t rdz = make_rsrc(gated ? (TIO *)o.dz + elem : nullptr,
                                                 gated ? bytes : 0);
    float *ldsB = lds;
    float *ldsC = lds + N * kLdsStride;
#pragma unroll
    for (int i = TT - 1; i >= 0; --i) {
        const bool valid = i < rows;
        RowRaw<N, TIO> brow, crow;
        const int64_t row = c.bL + (valid ? t0 + i : t0);
        fetch_row(brow, Bm, row);
        fetch_row(crow, Cm, row);
        const float ut = raw_f<TIO>(ch.u[i]);
        const float xr = raw_f<TIO>(ch.x[i]) + c.bias;
        const float sp = softplus(xr);
        float dt = c.softplus ? sp : xr;
        dt = valid ? dt : 0.0f;
        const float du = dt * ut;
        const float zt = raw_f<TIO>(ch.z[i]);
        const float dyt = raw_f<TIO>(ch.dy[i]);
        const float sz = sigmoid(zt);
        const float gz = gated ? zt * sz : 1.0f;
        const float dypre = dyt * gz;
        // factors of the dB, dC terms, zero on lanes past dim (they add nothing)
        const float du_a = active ? du : 0.0f;
        const float dypre_a = active ? dypre : 0.0f;
        const float r = POW ? hw_exp2(dt * c.A2_0) : 0.0f;
        float pw = 1.0f;
        float ypre = c.Dd * ut, sLB = 0.0f, wA = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float Bn = row_val<N>(brow, n), Cn = row_val<N>(crow, n);
            const float hn = hs[i][n];
            const float lam = fmaf(Cn, dypre, g[n]);
            ypre = fmaf(Cn, hn, ypre);
            const float q = fmaf(-du, Bn, hn);        // A_bar_t h_{t-1}
            const float wq = lam * q;
            wA = fmaf(POW ? (float)(n + 1) : A2[n], wq, wA);
            dA[n] = fmaf(dt, wq, dA[n]);
            sLB = fmaf(lam, Bn, sLB);
            // this lane's terms of dB_t[n] and dC_t[n]; row n of the LDS tiles
            ldsB[n * kLdsStride + lane] = lam * du_a;
            ldsC[n * kLdsStride + lane] = dypre_a * hn;
            const float a = POW ? (pw *= r) : hw_exp2(dt * A2[n]);
            g[n] = a * lam;
        }
        // sum_n A[n] w[n]: A2 carries log2(e), the structured chain A[d,0]
        const float dDelta = (POW ? wA * c.A2_0 : wA) * kLn2 + ut * sLB;
        const float dut = dypre * c.Dd + dt * sLB;
        const float ddl = valid ? (c.softplus ? dDelta * sigmoid(xr) : dDelta) : 0.0f;
        dD = fmaf(dypre, ut, dD);   // dy = 0 on padding steps
        dbias += ddl;
        const int soff = i * c.row_bytes;
        buf_store(rdu, c.voff_store, soff, dut, (TIO *)nullptr);
        buf_store(rdd, c.voff_store, soff, ddl, (TIO *)nullptr);
        if (gated) {
            const float dz = dyt * ypre * sz * (1.0f + zt * (1.0f - sz));
            buf_store(rdz, c.voff_store, soff, dz, (TIO *)nullptr);
        }
        // dB_t[n], dC_t[n] summed over the wave's 64 channels: 64/N lanes share
        // row n, each adds N entries, then xor-shuffles combine the shares.
        __syncthreads();
        const int nl = lane % N, share = lane / N;
        float sb = 0.0f, sc = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            sb += ldsB[nl * kLdsStride + share * N + j];
            sc += ldsC[nl * kLdsStride + share * N + j];
        }
#pragma unroll
        for (int m = N; m < kLanes; m <<= 1) {
            sb += __shfl_xor(sb, m);
            sc += __shfl_xor(sc, m);
        }
        __syncthreads();
        if (lane < N && valid) {
            const int64_t off = ((grp_in_row * batch + c.b) * c.L + t0 + i) * N + lane;
            o.pB[off] = sb;
            o.pC[off] = sc;
        }
    }
}

template <int N, bool POW, typename TIO>
__device__ __forceinline__ void bwd_part(const TIO *u, const TIO *delta, const TIO *z,
                                         const TIO *dy, const TIO *Bm, const TIO *Cm,
                                         const WaveCtx &c, const float *ck, const float (&A2)[N],
                                         float (&g)[N], float (&dA)[N], float &dD, float &dbias,
                                         const BwdOut &o, int64_t grp_in_row, int64_t batch,
                                         float *lds, int lane, bool active)
{
    const bool gated = z != nullptr;
    const int64_t nchunks = (c.l_end - c.l_begin + TT - 1) / TT;
    int64_t t0 = c.l_begin + (nchunks - 1) * TT;
    BwdChunk A, B;
    load_bwd_chunk(A, u, delta, z, dy, c, t0, true);
    for (;;) {
        load_bwd_chunk(B, u, delta, z, dy, c, t0 - TT, true);
        bwd_chunk<N, POW>(A, Bm, Cm, c, t0, ck + (t0 / TT) * (N * kLanes), A2, g, dA, dD, dbias,
                          gated, o, grp_in_row, batch, lds, lane, active);
        t0 -= TT;
        if (t0 < c.l_begin)
            break;
        A = B;
    }
}

// One wave per workgroup: the LDS transposes synchronise with __syncthreads.
template <int N, typename TIO>
__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(N <= 32 ? 2 : 1))) void bwd_main_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    const TIO *__restrict__ dy, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ dh_last,
    const float *__restrict__ asumm, const float *__restrict__ ckpt, BwdOut o, int64_t L,
    int64_t dim, int64_t batch, int64_t groups, int parts, int64_t part_len, int64_t nck)
{
    __shared__ float lds[2 * N * kLdsStride];
    WaveSetup w;
    if (!setup_wave(w, blockIdx.x, groups, parts, L, dim, part_len, (int)sizeof(TIO)))
        return;
    WaveCtx &c = w.c;
    c.softplus = delta_softplus;
    float A2[N];
    const bool pow_path = load_A<N>(A, w.d, A2, c.A2_0);
    c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
    c.Dd = D_skip ? D_skip[w.d] : 0.0f;
    // adjoint entering the part's last step from the right: dh_last folded
    // through the summaries of the later parts
    float g[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        g[n] = dh_last ? dh_last[(c.b * dim + w.d) * N + n] : 0.0f;
    // adjoint summary of part q is entry q - 1; fold parts P-1 down to part+1
    stream::fold_summaries<N>(g, asumm + (w.grp * (parts - 1)) * (N + 1) * kLanes + w.lane,
                              parts - 2, parts - 1 - w.part, -1, pow_path, A2, c.A2_0);
    float dA[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        dA[n] = 0.0f;
    float dD = 0.0f, dbias = 0.0f;
    const int64_t groups_per_row = (dim + kLanes - 1) / kLanes;
    const int64_t gir = w.grp % groups_per_row;
    const float *ck = ckpt + w.grp * nck * (N * kLanes) + w.lane;
    if (pow_path)
        bwd_part<N, true>(u, delta, z, dy, Bm, Cm, c, ck, A2, g, dA, dD, dbias, o, gir, batch,
                          lds, w.lane, w.active);
    else
        bwd_part<N, false>(u, delta, z, dy, Bm, Cm, c, ck, A2, g, dA, dD, dbias, o, gir, batch,
                           lds, w.lane, w.active);
    if (w.active) {
        const int64_t slot = c.b * parts + w.part;
#pragma unroll
        for (int n = 0; n < N; ++n)
            o.pA[(slot * dim + w.d) * N + n] = dA[n];
        o.pD[slot * dim + w.d] = dD;
        o.pbias[slot * dim + w.d] = dbias;
        if (w.part == 0 && o.dh0) {
#pragma unroll
            for (int n = 0; n < N; ++n)
                o.dh0[(c.b * dim + w.d) * N + n] = g[n];
        }
    }
}

// ---------------------------------------------------------------------------
// 5. reductions of the partials (fixed order)
// ---------------------------------------------------------------------------
// out[i] = sum_k in[k * P + i] for i < P, k < K: a block of four waves owns 64
// columns; wave w adds the rows k = w, w + 4, ... (eight loads in flight),
// then the four sums are added in wave order.
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const float *__restrict__ in,
                                                         float *__restrict__ out, int64_t P,
                                                         int64_t K)
{
    __shared__ float part[4][kLanes];
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * kLanes + lane;
    float s = 0.0f;
    if (i < P) {
        int64_t k = wave;
        for (; k + 28 < K; k += 32) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = in[(k + 4 * j) * P + i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s += v[j];
        }
        for (; k < K; k += 4)
            s += in[k * P + i];
    }
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && i < P)
        out[i] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

hipError_t launch_colsum(const float *in, float *out, int64_t P, int64_t K, hipStream_t s)
{
    if (!out || P <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(bwd_colsum_kernel, dim3((unsigned)((P + kLanes - 1) / kLanes)), dim3(256),
                       0, s, in, out, P, K);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// workspace and launch
// ---------------------------------------------------------------------------
struct BwdLayout {
    StreamPlan p;
    int64_t nck, gpr;
    size_t fsumm, asumm, ckpt, pB, pC, pA, pD, pbias, total;   // byte offsets
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    BwdLayout w;
    w.p = make_stream_plan(batch, L, dim);
    w.nck = (L + TT - 1) / TT;
    w.gpr = (dim + kLanes - 1) / kLanes;
    const size_t summ = (size_t)w.p.groups * (w.p.parts > 1 ? w.p.parts - 1 : 0) * (N + 1) *
                        kLanes * 4;
    size_t off = 0;
    w.fsumm = off; off = align256(off + summ);
    w.asumm = off; off = align256(off + summ);
    w.ckpt = off; off = align256(off + (size_t)w.p.groups * w.nck * N * kLanes * 4);
    w.pB = off; off = align256(off + (size_t)w.gpr * batch * L * N * 4);
    w.pC = off; off = align256(off + (size_t)w.gpr * batch * L * N * 4);
    w.pA = off; off = align256(off + (size_t)batch * w.p.parts * dim * N * 4);
    w.pD = off; off = align256(off + (size_t)batch * w.p.parts * dim * 4);
    w.pbias = off; off = align256(off + (size_t)batch * w.p.parts * dim * 4);
    w.total = off + 256;   // room to align the base
    return w;
}

template <int N, typename TIO>
hipError_t launch_bwd_n(const BwdArgs &a, hipStream_t s)
{
    const BwdLayout w = bwd_layout(a.fwd.batch, a.fwd.L, a.fwd.dim, N);
    char *base = (char *)(((uintptr_t)a.fwd.workspace + 255) & ~(uintptr_t)255);
    float *fsumm = (float *)(base + w.fsumm), *asumm = (float *)(base + w.asumm);
    float *ckpt = (float *)(base + w.ckpt);
    BwdOut o;
    o.du = a.du; o.ddelta = a.ddelta; o.dz = a.dz;
    o.pB = (float *)(base + w.pB); o.pC = (float *)(base + w.pC);
    o.pA = (float *)(base + w.pA); o.pD = (float *)(base + w.pD);
    o.pbias = (float *)(base + w.pbias);
    o.dh0 = a.dh0;
    const StreamPlan &p = w.p;
    hipError_t e;
    if (p.parts > 1) {
        e = launch_fwd_summaries(a.fwd, p, fsumm, s);
        if (e != hipSuccess)
            return e;
        const int64_t waves = p.groups * (p.parts - 1);
        hipLaunchKernelGGL((bwd_adjoint_summary_kernel<N, TIO>), dim3((unsigned)((waves + 3) / 4)),
                           dim3(kLanes * 4), 0, s, (const TIO *)a.fwd.delta, (const TIO *)a.fwd.z,
                           (const TIO *)a.dy, a.fwd.A, (const TIO *)a.fwd.Cm, a.fwd.delta_bias,
                           a.fwd.delta_softplus, asumm, a.fwd.L, a.fwd.dim, p.groups, p.parts, p.part_len);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    const int64_t waves = p.groups * p.parts;
    hipLaunchKernelGGL((bwd_checkpoint_kernel<N, TIO>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(kLanes * 4), 0, s, (const TIO *)a.fwd.u, (const TIO *)a.fwd.delta,
                       a.fwd.A, (const TIO *)a.fwd.Bm, a.fwd.delta_bias, a.fwd.delta_softplus,
                       a.fwd.h0, fsumm, ckpt, a.fwd.L, a.fwd.dim, p.groups, p.parts, p.part_len, w.nck);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((bwd_main_kernel<N, TIO>), dim3((unsigned)waves), dim3(kLanes), 0, s,
                       (const TIO *)a.fwd.u, (const TIO *)a.fwd.delta, (const TIO *)a.fwd.z,
                       (const TIO *)a.dy, a.fwd.A, (const TIO *)a.fwd.Bm, (const TIO *)a.fwd.Cm,
                       a.fwd.D_skip, a.fwd.delta_bias, a.fwd.delta_softplus, a.dh_last, asumm,
                       ckpt, o, a.fwd.L, a.fwd.dim, a.fwd.batch, p.groups, p.parts, p.part_len, w.nck);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t count = a.fwd.batch * a.fwd.L * N;
    const int64_t slots = a.fwd.batch * p.parts;
    if ((e = launch_colsum(o.pB, a.dB, count, w.gpr, s)) != hipSuccess ||
        (e = launch_colsum(o.pC, a.dC, count, w.gpr, s)) != hipSuccess ||
        (e = launch_colsum(o.pA, a.dA, a.fwd.dim * N, slots, s)) != hipSuccess ||
        (e = launch_colsum(o.pD, a.dD, a.fwd.dim, slots, s)) != hipSuccess ||
        (e = launch_colsum(o.pbias, a.ddelta_bias, a.fwd.dim, slots, s)) != hipSuccess)
        return e;
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s)
{
    switch (a.fwd.N) {
    case 4: return launch_bwd_n<4, TIO>(a, s);
    case 8: return launch_bwd_n<8, TIO>(a, s);
    case 16: return launch_bwd_n<16, TIO>(a, s);
    case 32: return launch_bwd_n<32, TIO>(a, s);
    case 64: return launch_bwd_n<64, TIO>(a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    return bwd_layout(batch, L, dim, N).total;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream)
{
    return a.fwd.dtype == 1 ? launch_bwd_t<uint16_t>(a, stream) : launch_bwd_t<float>(a, stream);
}

} // namespace selscan
