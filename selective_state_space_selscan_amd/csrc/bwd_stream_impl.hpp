// Backward of the selective scan for gfx950, with recomputation: kernel
// templates shared by the five instantiations (bwd_stream.hip: Euler B_bar,
// forward direction, with the addressing fixed at compile time;
// bwd_stream_rev.hip: the same in reverse; bwd_stream_zoh.hip,
// bwd_stream_conv.hip, bwd_stream_zoh_conv.hip: either direction, chosen at
// run time).
//
// Gradients of y = (C_t.h_t + D u_t) * SiLU(z_t), h_t = exp(Delta_t A) h_{t-1}
// + B_bar_t u_t for an upstream dy (and optionally dh_last).  The states are
// not stored by the forward: they are recomputed here (Gu & Dao deep-reading
// report §2.4; selection-mechanism article discosf.com §3.4).  The adjoint
// lambda_t = dL/dh_t runs backwards,
//   lambda_t = C_t dypre_t + A_bar_{t+1} lambda_{t+1},   dypre_t = dy_t SiLU(z_t),
// and every gradient is a per-step product of lambda_t, h_t and the inputs.
//
// Layout as in the streaming forward: lane = channel of a 64-channel group,
// wave = (group, sequence part), parts from the forward's plan.  Pipeline:
//   1. forward part summaries (the forward's summary pass);
//   2. adjoint part summaries, for the fold from the right: over a part
//      [s, e), the adjoint leaving it to the left is
//        g_{s-1} = sum_t (prod_{k=s..t} A_bar_k) C_t dypre_t
//        + exp(A sum_part Delta) g_{e-1},
//      the same associative operator as the forward, in reverse; the carry
//      kernel of the forward then folds h0 from the left and dh_last from
//      the right into the entry state of every part, both directions;
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
//
// Variants (those of the forward, fwd_stream_impl.hpp).  All passes run in
// scan order s; they differ only where the step's input or B_bar enters:
//   * reverse direction: scan step s is timestep L-1-s (addressing only; h0
//     enters before scan step 0 and dh_last is the gradient of the state
//     after the last scan step).
//   * exact zero-order hold: B_bar_n = c_n B_n with c_n = (e_n - 1) / a_n,
//     e_n = exp(Delta a_n).  Then dc_n/dDelta = e_n and
//     dc_n/da_n = (Delta e_n - c_n) / a_n, which is Delta^2 times the series
//     1/2 + x/3 + x^2/8 + x^3/30 + x^4/144 + x^5/840 + x^6/5760 in x = Delta a_n
//     (the coefficients (m-1)/m! of x^m in x e^x - e^x + 1) where |x| is small.
//   * conv1d + SiLU prologue: the scan input is u_s = SiLU(p_s) with
//     p_s = b + sum_m w_m x_{s-3+m} (taps zero-padded in front to 4).  With
//     gu_s the gradient of u_s and gp_s = gu_s SiLU'(p_s):
//       dx_{s'} = sum_m w_m gp_{s'+3-m},  dw_m = sum_s gp_s x_{s-3+m},
//       db = sum_s gp_s.
//     dx_s needs gp of the steps s..s+3: the wave keeps the contributions of
//     the three later steps in a register ring.  For the last three steps of
//     a part (but the last), the later steps belong to the next part's wave:
//     both partial sums go to the workspace and a fix-up pass adds them.
#pragma once

#include "fwd_stream_impl.hpp"

namespace selscan {
namespace bwd {

using stream::ExtParams;
using stream::kLanes;
using stream::kMaxConv;
using stream::kVarConv;
using stream::kVarExt;
using stream::kVarRev;
using stream::kVarZoh;
using stream::RowRaw;
using stream::TT;
using stream::WaveCtx;
using stream::fetch_row;
using stream::row_dir;
using stream::row_val;
using stream::run_t_lo;
using stream::scan_row;
using stream::step_soff;

constexpr int kLdsStride = kLanes + 1;  // padded rows: conflict-free LDS transposes
constexpr int kHalo = kMaxConv - 1;     // conv window: steps before a step
static_assert(TT >= kHalo, "the conv window must fit in the chunk before");

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
                                           int64_t part_len, int elem_bytes, int rev)
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
    c.rev = rev;
    c.softplus = 0;
    c.invA0 = 0.0f;
    c.cb = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j)
        c.cw[j] = 0.0f;
    return true;
}

// A2 = A log2(e) of this lane's channel (and 1/A for the exact ZOH); true
// when A[d,n] = (n+1) A[d,0] holds for every lane of the wave (the
// structured power chain applies).
template <int N, bool ZOH>
__device__ __forceinline__ bool load_A(const float *A, int64_t d, float (&A2)[N], float (&invA)[N],
                                       WaveCtx &c)
{
    const float A0 = A[d * N];
    bool structured = true;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        invA[n] = ZOH ? 1.0f / an : 0.0f;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    c.A2_0 = A0 * kLog2e;
    c.invA0 = invA[0];
    return __all(structured);
}

__device__ __forceinline__ float sigmoid(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

template <typename TIO>
__device__ __forceinline__ float raw_f(uint32_t v) { return raw_to_f32(v, tag<TIO>()); }

// d c / d a of the exact-ZOH coefficient c = (e - 1) / a, e = exp(Delta a),
// given x2 = Delta a log2(e): (Delta e - c) / a, or where that cancels
// (|x2| < 1/2) Delta^2 times the degree-6 series above (truncation below
// 1e-6 relative there).  a = 0 takes the series: Delta^2 / 2.
__device__ __forceinline__ float zoh_dcoeff(float dt, float x2, float e, float c, float inv_a)
{
    const float x = x2 * kLn2;
    float p = fmaf(x, 1.0f / 5760.0f, 1.0f / 840.0f);
    p = fmaf(x, p, 1.0f / 144.0f);
    p = fmaf(x, p, 1.0f / 30.0f);
    p = fmaf(x, p, 1.0f / 8.0f);
    p = fmaf(x, p, 1.0f / 3.0f);
    p = fmaf(x, p, 0.5f);
    const float series = dt * dt * p;
    const float direct = fmaf(dt, e, -c) * inv_a;
    return fabsf(x2) < 0.5f ? series : direct;
}

// Inputs of TT steps for the backward: u (the raw input x with the conv
// prologue), Delta_raw, z, dy (raw bits).
struct BwdChunk {
    uint32_t u[TT], x[TT], z[TT], dy[TT];
};

// Loads the chunk at scan step t0.  Chunks past the part's end, or starting
// below `lo` (the part's start, or the chunk before it for the conv window),
// read nothing (zeros).
template <int VAR, typename TIO>
__device__ __forceinline__ void load_bwd_chunk(BwdChunk &ch, const TIO *u, const TIO *delta,
                                               const TIO *z, const TIO *dy, const WaveCtx &c,
                                               int64_t t0, bool with_u, int64_t lo)
{
    int64_t rows = c.l_end - t0;
    rows = rows < 0 ? 0 : (rows > TT ? TT : rows);
    if (t0 < lo)
        rows = 0;
    const int64_t elem = (c.bL + run_t_lo<VAR>(c, t0, rows)) * c.dim + c.d0;
    const int64_t bytes = rows > 0 ? (rows * c.dim - c.d0) * (int64_t)sizeof(TIO) : 0;
    const int64_t safe = rows > 0 ? elem : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(delta + safe, bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(dy + safe, bytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(with_u ? u + safe : nullptr, with_u ? bytes : 0);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z ? z + safe : nullptr, z ? bytes : 0);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int soff = step_soff<VAR>(c, i, (int)rows);
        ch.x[i] = buf_load_raw(rx, c.voff, soff, delta);
        ch.dy[i] = buf_load_raw(ry, c.voff, soff, dy);
        ch.u[i] = buf_load_raw(ru, c.voff, soff, u);
        ch.z[i] = buf_load_raw(rz, c.voff, soff, z);
    }
}

// ---------------------------------------------------------------------------
// 2. adjoint part summaries (parts 1 .. P-1)
// ---------------------------------------------------------------------------
// Walks the part forwards: with Pr_t[n] = prod_{k=s..t} A_bar_k[n],
// v[n] = sum_t Pr_t[n] C_t[n] dypre_t.  For structured A, Pr_t[n] = P_t^(n+1)
// with P_t the running product of r_k = exp(Delta_k A[d,0]): a multiply and an
// FMA per (t, n), as in the forward summary.  The adjoint recurrence does not
// involve B_bar or the step input, so the variants share it.
template <int N, bool POW, int VAR, typename TIO>
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
    const int64_t dir = row_dir<VAR>(c);
    load_bwd_chunk<VAR>(A, (const TIO *)nullptr, delta, z, dy, c, t0, false, c.l_begin);
    for (;;) {
        load_bwd_chunk<VAR>(B, (const TIO *)nullptr, delta, z, dy, c, t0 + TT, false, c.l_begin);
        const int rows = (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
        const int64_t row0 = scan_row<VAR>(c, t0);
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            if (i >= rows)
                break;   // uniform: only the sequence end is partial
            RowRaw<N, TIO> crow;
            fetch_row(crow, Cm, row0 + i * dir);
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

template <int N, int VAR, typename TIO>
__device__ __forceinline__ void adjoint_summary_wave(
    const TIO *__restrict__ delta, const TIO *__restrict__ z, const TIO *__restrict__ dy,
    const float *__restrict__ A, const TIO *__restrict__ Cm, const float *__restrict__ delta_bias,
    int delta_softplus, float *__restrict__ asumm, int rev, int64_t blk, int64_t L, int64_t dim,
    int64_t groups, int parts, int64_t part_len)
{
    WaveSetup w;
    const int64_t gw = blk * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (!setup_wave(w, gw, groups, parts - 1, L, dim, part_len, (int)sizeof(TIO), rev))
        return;
    // wave (grp, q) summarises part q + 1
    w.part += 1;
    WaveCtx &c = w.c;
    c.l_begin = (int64_t)w.part * part_len;
    c.l_end = c.l_begin + part_len < L ? c.l_begin + part_len : L;
    c.softplus = delta_softplus;
    float A2[N], invA[N];
    const bool pow_path = load_A<N, false>(A, w.d, A2, invA, c);
    c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
    float v[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        v[n] = 0.0f;
    float sdelta = 0.0f;
    if (pow_path)
        adjoint_summary_part<N, true, VAR>(delta, z, dy, Cm, c, A2, v, sdelta);
    else
        adjoint_summary_part<N, false, VAR>(delta, z, dy, Cm, c, A2, v, sdelta);
    float *o = asumm + ((w.grp * (parts - 1) + (w.part - 1)) * (N + 1)) * kLanes + w.lane;
    o[0] = sdelta;
#pragma unroll
    for (int n = 0; n < N; ++n)
        o[(n + 1) * kLanes] = v[n];
}

// ---------------------------------------------------------------------------
// 3. checkpoints: the state entering every TT-step chunk
// ---------------------------------------------------------------------------
template <int N, bool POW, bool SP, int VAR, typename TIO>
__device__ __forceinline__ void checkpoint_part(const TIO *__restrict__ u,
                                                const TIO *__restrict__ delta,
                                                const TIO *__restrict__ Bm, const WaveCtx &c,
                                                const float (&A2)[N], const float (&invA)[N],
                                                float (&h)[N], float *__restrict__ ck,
                                                float (&win)[kHalo])
{
    float sdelta = 0.0f;
    stream::Chunk A, B;
    int64_t t0 = c.l_begin;
    stream::load_chunk<false, VAR>(A, u, delta, (const TIO *)nullptr, c, t0);
    for (;;) {
        stream::load_chunk<false, VAR>(B, u, delta, (const TIO *)nullptr, c, t0 + TT);
        float *o = ck + (t0 / TT) * (N * kLanes);
#pragma unroll
        for (int n = 0; n < N; ++n)
            o[n * kLanes] = h[n];
        stream::run_any_chunk<N, true, false, SP, POW, VAR>(A, Bm, Bm, (TIO *)nullptr, c, t0,
                                                            A2, invA, h, sdelta, win);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
        A = B;
    }
}

// Passes 2 and 3 in one launch (ROLES = 3): the adjoint summaries
// (arithmetic-bound) and the checkpoints (bound by their stores) are
// independent, and sharing the CUs lets one's arithmetic overlap the other's
// memory traffic: 3.6 % off the plain backward and 2 % off the conv4 one,
// measured.  Blocks alternate between the roles while both have work left.
// ROLES = 1 or 2: one role alone (the exact-ZOH variants, whose heavier
// checkpoint walk sets the registers of both roles: 0.6 % slower merged with
// reverse and conv4, no gain without).
template <int N, int VAR, int ROLES, typename TIO>
__global__ __launch_bounds__(kLanes * 4) void bwd_pass23_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    const TIO *__restrict__ dy, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ delta_bias, int delta_softplus,
    const float *__restrict__ h0, const float *__restrict__ fentry, float *__restrict__ asumm,
    float *__restrict__ ckpt, int64_t nck, ExtParams ext, int64_t L, int64_t dim, int64_t groups,
    int parts, int64_t part_len, int64_t adj_blocks, int64_t ck_blocks)
{
    const int64_t bid = blockIdx.x;
    bool is_adj = ROLES == 1;
    int64_t idx = bid;
    if constexpr (ROLES == 3) {
        const int64_t m = adj_blocks < ck_blocks ? adj_blocks : ck_blocks;
        if (bid < 2 * m) {
            is_adj = (bid & 1) == 0;
            idx = bid >> 1;
        } else {
            is_adj = adj_blocks > ck_blocks;
            idx = m + (bid - 2 * m);
        }
    }
    if constexpr ((ROLES & 1) != 0) {
        if (is_adj) {
            adjoint_summary_wave<N, (VAR & ~kVarRev) == 0 ? VAR : (int)kVarExt, TIO>(
                delta, z, dy, A, Cm, delta_bias, delta_softplus, asumm, ext.rev, idx, L, dim,
                groups, parts, part_len);
            return;
        }
    }
    // the checkpoint role, written out here: as an inlined function the
    // compiler schedules it differently and the conv variants need 149
    // VGPRs instead of 123 at N = 16 (3 waves per SIMD instead of 4)
    if constexpr ((ROLES & 2) != 0) {
        if (is_adj)
            return;
        constexpr bool ZOH = (VAR & kVarZoh) != 0;
        constexpr bool CONV = (VAR & kVarConv) != 0;
        WaveSetup w;
        const int64_t gw = idx * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (!setup_wave(w, gw, groups, parts, L, dim, part_len, (int)sizeof(TIO), ext.rev))
            return;
        WaveCtx &c = w.c;
        c.softplus = delta_softplus;
        float A2[N], invA[N];
        const bool pow_path = load_A<N, ZOH>(A, w.d, A2, invA, c);
        c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
        c.Dd = 0.0f;
        float win[kHalo];
#pragma unroll
        for (int j = 0; j < kHalo; ++j)
            win[j] = 0.0f;
        if constexpr (CONV) {
            stream::conv_taps(c, ext, w.d);
            stream::conv_window<VAR>(win, c, u, w.d);
        }
        // entry state: h0 carried through the earlier parts (fentry, null when
        // the sequence is not split)
        float h[N];
        if (fentry) {
            stream::load_entry<N>(h, fentry, w.grp, parts, w.part, w.lane);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n)
                h[n] = h0 ? h0[(c.b * dim + w.d) * N + n] : 0.0f;
        }
        float *ck = ckpt + w.grp * nck * (N * kLanes) + w.lane;
        // with kVarExt the softplus switch is read at run time (SP unused)
        const bool sp = (VAR & kVarExt) != 0 || delta_softplus;
        if (pow_path) {
            if (sp) checkpoint_part<N, true, true, VAR>(u, delta, Bm, c, A2, invA, h, ck, win);
            else checkpoint_part<N, true, false, VAR>(u, delta, Bm, c, A2, invA, h, ck, win);
        } else {
            if (sp) checkpoint_part<N, false, true, VAR>(u, delta, Bm, c, A2, invA, h, ck, win);
            else checkpoint_part<N, false, false, VAR>(u, delta, Bm, c, A2, invA, h, ck, win);
        }
    }
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
    // conv prologue only
    float *pW;          // (batch, parts, dim, conv_k) partial sums of dconv_w
    float *pWb;         // (batch, parts, dim) partial sums of dconv_b
    float *xown;        // (groups, parts, kHalo, 64): dx of a part's last kHalo steps, own share
    float *xcarry;      // (groups, parts, kHalo, 64): a part's share of the kHalo steps before it
};

// Per-wave running sums of the main pass.
struct BwdAcc {
    float dD, dbias;
    float dcw[kMaxConv], dcb;   // conv prologue
    float ring[kHalo];          // conv: shares of dx of the kHalo steps before the current one
};

// TT steps: states recomputed from the chunk's checkpoint, then the adjoint
// steps from the last to the first.  prev: the chunk before (its raw inputs
// are the conv window; unused without the conv prologue).
template <int N, bool POW, int VAR, typename TIO>
__device__ __forceinline__ void bwd_chunk(const BwdChunk &ch, const BwdChunk &prev, const TIO *Bm,
                                          const TIO *Cm, const WaveCtx &c, int64_t t0,
                                          const float *ck, const float (&A2)[N],
                                          const float (&invA)[N], float (&g)[N], float (&dA)[N],
                                          BwdAcc &acc, bool gated, const BwdOut &o,
                                          int64_t grp_in_row, int64_t batch, float *lds, int lane,
                                          bool active, float *xown)
{
    constexpr bool ZOH = (VAR & kVarZoh) != 0;
    constexpr bool CONV = (VAR & kVarConv) != 0;
    // Two equivalent forms of the per-step addressing and ordering, each the
    // faster one (fewer scalar-register spills, measured) for its case: with
    // the direction fixed at compile time, rows and inputs are formed at use;
    // with a run-time direction, from a row base and step computed once.
    // (kVarRev: the fixed direction is the reverse one.)
    constexpr bool FIXED = (VAR & kVarExt) == 0;
    constexpr bool REVF = (VAR & kVarRev) != 0;
    const int rows = (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    const int64_t row0 = scan_row<VAR>(c, t0);
    const int64_t dir = row_dir<VAR>(c);
    auto step_row = [&](int i, bool valid) -> int64_t {
        if constexpr (FIXED) {
            const int64_t st = valid ? t0 + i : t0;
            return c.bL + (REVF ? c.L - 1 - st : st);
        } else {
            return valid ? row0 + i * dir : row0;
        }
    };
    // scan inputs of the TT steps; with the conv prologue, the raw inputs of
    // steps t0-kHalo .. t0+TT-1 (xw[j] is step t0-kHalo+j) and the
    // pre-activations
    float xw[kHalo + TT], us[TT], pre[TT];
#pragma unroll
    for (int j = 0; j < kHalo; ++j)
        xw[j] = CONV ? raw_f<TIO>(prev.u[TT - kHalo + j]) : 0.0f;
#pragma unroll
    for (int i = 0; i < TT; ++i)
        xw[kHalo + i] = raw_f<TIO>(ch.u[i]);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        if constexpr (CONV) {
            float a = c.cb;
#pragma unroll
            for (int m = 0; m < kMaxConv; ++m)
                a = fmaf(c.cw[m], xw[i + m], a);
            pre[i] = a;
            us[i] = silu(a);
        } else {
            pre[i] = 0.0f;
            us[i] = xw[kHalo + i];
        }
    }
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
            fetch_row(brow, Bm, step_row(i, i < rows));
            const float ut = (FIXED && !CONV) ? raw_f<TIO>(ch.u[i]) : us[i];
            const float xr = raw_f<TIO>(ch.x[i]) + c.bias;
            const float sp = softplus(xr);
            float dt = c.softplus ? sp : xr;
            dt = i < rows ? dt : 0.0f;
            const float du = dt * ut;
            const float r = POW ? hw_exp2(dt * c.A2_0) : 0.0f;
            float pw = 1.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float x2 = dt * A2[n];
                const float a = POW ? (pw *= r) : hw_exp2(x2);
                const float bu = ZOH ? stream::zoh_coeff(dt, x2, a, invA[n]) *
                                           (ut * row_val<N>(brow, n))
                                     : du * row_val<N>(brow, n);
                h[n] = fmaf(a, h[n], bu);
                hs[i][n] = h[n];
            }
        }
    }
    // adjoint steps
    const int64_t elem = (c.bL + run_t_lo<VAR>(c, t0, rows)) * c.dim + c.d0;
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
        const int64_t row = step_row(i, valid);
        fetch_row(brow, Bm, row);
        fetch_row(crow, Cm, row);
        const float ut = (FIXED && !CONV) ? raw_f<TIO>(ch.u[i]) : us[i];
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
        const float ut_a = active ? ut : 0.0f;
        const float dypre_a = active ? dypre : 0.0f;
        const float r = POW ? hw_exp2(dt * c.A2_0) : 0.0f;
        float pw = 1.0f;
        float ypre = c.Dd * ut, sLB = 0.0f, wA = 0.0f, wE = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float Bn = row_val<N>(brow, n), Cn = row_val<N>(crow, n);
            const float hn = hs[i][n];
            const float lam = fmaf(Cn, dypre, g[n]);
            ypre = fmaf(Cn, hn, ypre);
            float a = 0.0f;
            if constexpr (ZOH || !FIXED)
                a = POW ? (pw *= r) : hw_exp2(dt * A2[n]);
            if constexpr (ZOH) {
                const float x2 = dt * A2[n];
                const float cn = stream::zoh_coeff(dt, x2, a, invA[n]);
                const float lb = lam * Bn;
                const float q = fmaf(-cn, ut * Bn, hn);   // A_bar_t h_{t-1}
                const float wq = lam * q;
                wA = fmaf(A2[n], wq, wA);
                wE = fmaf(a, lb, wE);
                dA[n] = fmaf(dt, wq, fmaf(zoh_dcoeff(dt, x2, a, cn, invA[n]), lb * ut, dA[n]));
                sLB = fmaf(cn, lb, sLB);
                ldsB[n * kLdsStride + lane] = lam * (cn * ut_a);
            } else {
                const float q = fmaf(-du, Bn, hn);        // A_bar_t h_{t-1}
                const float wq = lam * q;
                wA = fmaf(POW ? (float)(n + 1) : A2[n], wq, wA);
                dA[n] = fmaf(dt, wq, dA[n]);
                sLB = fmaf(lam, Bn, sLB);
                ldsB[n * kLdsStride + lane] = lam * du_a;
            }
            // this lane's terms of dC_t[n]; row n of the LDS tiles
            ldsC[n * kLdsStride + lane] = dypre_a * hn;
            if constexpr (!ZOH && FIXED)
                a = POW ? (pw *= r) : hw_exp2(dt * A2[n]);
            g[n] = a * lam;
        }
        // sum_n A[n] w[n]: A2 carries log2(e), the structured chain A[d,0]
        float dDelta, dut;
        if constexpr (ZOH) {
            dDelta = wA * kLn2 + ut * wE;
            dut = fmaf(dypre, c.Dd, sLB);
        } else {
            dDelta = (POW ? wA * c.A2_0 : wA) * kLn2 + ut * sLB;
            dut = dypre * c.Dd + dt * sLB;
        }
        const float ddl = valid ? (c.softplus ? dDelta * sigmoid(xr) : dDelta) : 0.0f;
        acc.dD = fmaf(dypre, ut, acc.dD);   // dy = 0 on padding steps
        acc.dbias += ddl;
        const int soff = step_soff<VAR>(c, i, rows);
        int soff_du = soff;
        float dxo = dut;
        if constexpr (CONV) {
            // through SiLU'(p) = s (1 + p (1 - s)), s = sigmoid(p), and the taps
            const float sa = sigmoid(pre[i]);
            const float gp = valid ? dut * (sa * fmaf(pre[i], 1.0f - sa, 1.0f)) : 0.0f;
            acc.dcb += gp;
#pragma unroll
            for (int m = 0; m < kMaxConv; ++m)
                acc.dcw[m] = fmaf(gp, xw[i + m], acc.dcw[m]);
            dxo = fmaf(c.cw[kMaxConv - 1], gp, acc.ring[0]);
#pragma unroll
            for (int j = 0; j < kHalo - 1; ++j)
                acc.ring[j] = fmaf(c.cw[kMaxConv - 2 - j], gp, acc.ring[j + 1]);
            acc.ring[kHalo - 1] = c.cw[0] * gp;
            // the last kHalo steps of a part followed by another: share to the workspace
            const int64_t s = t0 + i;
            if (xown && valid && s >= c.l_end - kHalo) {
                xown[(c.l_end - 1 - s) * kLanes] = dxo;
                soff_du = stream::kStoreOffsetOutOfRange;
            }
        }
        buf_store(rdu, c.voff_store, soff_du, dxo, (TIO *)nullptr);
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
            const int64_t t = FIXED ? (REVF ? c.L - 1 - (t0 + i) : t0 + i)
                                    : row - c.bL;   // timestep of the step
            const int64_t off = ((grp_in_row * batch + c.b) * c.L + t) * N + lane;
            o.pB[off] = sb;
            o.pC[off] = sc;
        }
    }
}

template <int N, bool POW, int VAR, typename TIO>
__device__ __forceinline__ void bwd_part(const TIO *u, const TIO *delta, const TIO *z,
                                         const TIO *dy, const TIO *Bm, const TIO *Cm,
                                         const WaveCtx &c, const float *ck, const float (&A2)[N],
                                         const float (&invA)[N], float (&g)[N], float (&dA)[N],
                                         BwdAcc &acc, const BwdOut &o, int64_t grp_in_row,
                                         int64_t batch, float *lds, int lane, bool active,
                                         float *xown)
{
    constexpr bool CONV = (VAR & kVarConv) != 0;
    const bool gated = z != nullptr;
    const int64_t nchunks = (c.l_end - c.l_begin + TT - 1) / TT;
    int64_t t0 = c.l_begin + (nchunks - 1) * TT;
    BwdChunk A, B;
    if constexpr (CONV) {
        // The conv window of a chunk is in the chunk before it, so the loads
        // run two chunks ahead (that chunk has arrived when the window is
        // read); the chunk before the part is loaded for its window too.
        const int64_t lo = c.l_begin >= TT ? c.l_begin - TT : 0;
        BwdChunk C;
        load_bwd_chunk<VAR>(A, u, delta, z, dy, c, t0, true, lo);
        load_bwd_chunk<VAR>(B, u, delta, z, dy, c, t0 - TT, true, lo);
        for (;;) {
            load_bwd_chunk<VAR>(C, u, delta, z, dy, c, t0 - 2 * TT, true, lo);
            bwd_chunk<N, POW, VAR>(A, B, Bm, Cm, c, t0, ck + (t0 / TT) * (N * kLanes), A2, invA,
                                   g, dA, acc, gated, o, grp_in_row, batch, lds, lane, active,
                                   xown);
            t0 -= TT;
            if (t0 < c.l_begin)
                break;
            A = B;
            B = C;
        }
    } else {
        load_bwd_chunk<VAR>(A, u, delta, z, dy, c, t0, true, c.l_begin);
        for (;;) {
            load_bwd_chunk<VAR>(B, u, delta, z, dy, c, t0 - TT, true, c.l_begin);
            bwd_chunk<N, POW, VAR>(A, A, Bm, Cm, c, t0, ck + (t0 / TT) * (N * kLanes), A2, invA,
                                   g, dA, acc, gated, o, grp_in_row, batch, lds, lane, active,
                                   nullptr);
            t0 -= TT;
            if (t0 < c.l_begin)
                break;
            A = B;
        }
    }
}

// Main-pass occupancy: two waves per SIMD (256 VGPRs) up to N = 16; one
// (512 VGPRs, spills to AGPRs) from N = 32 on, where two waves spill 474
// VGPRs to scratch (batch 8, L 2048, D 1536, N 32: 4.35 -> 1.74 ms), and for
// the variants from N = 16 on, whose extra per-state terms would spill at 256.
template <int N, int VAR>
constexpr int bwd_waves_per_eu()
{
    if (N > 16)
        return 1;
    if ((VAR & (kVarZoh | kVarConv)) != 0 && N >= 16)
        return 1;
    return 2;
}

// One wave per workgroup: the LDS transposes synchronise with __syncthreads.
template <int N, int VAR, typename TIO>
__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu<N, VAR>()))) void bwd_main_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    const TIO *__restrict__ dy, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ dh_last,
    const float *__restrict__ aentry, const float *__restrict__ ckpt, BwdOut o, int64_t L,
    int64_t dim, int64_t batch, int64_t groups, int parts, int64_t part_len, int64_t nck,
    ExtParams ext)
{
    constexpr bool ZOH = (VAR & kVarZoh) != 0;
    constexpr bool CONV = (VAR & kVarConv) != 0;
    __shared__ float lds[2 * N * kLdsStride];
    WaveSetup w;
    if (!setup_wave(w, blockIdx.x, groups, parts, L, dim, part_len, (int)sizeof(TIO), ext.rev))
        return;
    WaveCtx &c = w.c;
    c.softplus = delta_softplus;
    float A2[N], invA[N];
    const bool pow_path = load_A<N, ZOH>(A, w.d, A2, invA, c);
    c.bias = delta_bias ? delta_bias[w.d] : 0.0f;
    c.Dd = D_skip ? D_skip[w.d] : 0.0f;
    if constexpr (CONV)
        stream::conv_taps(c, ext, w.d);
    // adjoint entering the part's last step from the right: dh_last folded
    // through the adjoint summaries of the later parts (aentry, null when the
    // sequence is not split)
    float g[N];
    if (aentry) {
        stream::load_entry<N>(g, aentry, w.grp, parts, w.part, w.lane);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n)
            g[n] = dh_last ? dh_last[(c.b * dim + w.d) * N + n] : 0.0f;
    }
    float dA[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        dA[n] = 0.0f;
    BwdAcc acc;
    acc.dD = acc.dbias = acc.dcb = 0.0f;
#pragma unroll
    for (int m = 0; m < kMaxConv; ++m)
        acc.dcw[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < kHalo; ++j)
        acc.ring[j] = 0.0f;
    const int64_t groups_per_row = (dim + kLanes - 1) / kLanes;
    const int64_t gir = w.grp % groups_per_row;
    const float *ck = ckpt + w.grp * nck * (N * kLanes) + w.lane;
    const int64_t wave_slot = w.grp * parts + w.part;
    float *xown = (CONV && w.part < parts - 1) ? o.xown + wave_slot * kHalo * kLanes + w.lane
                                               : nullptr;
    if (pow_path)
        bwd_part<N, true, VAR>(u, delta, z, dy, Bm, Cm, c, ck, A2, invA, g, dA, acc, o, gir, batch,
                               lds, w.lane, w.active, xown);
    else
        bwd_part<N, false, VAR>(u, delta, z, dy, Bm, Cm, c, ck, A2, invA, g, dA, acc, o, gir,
                                batch, lds, w.lane, w.active, xown);
    if constexpr (CONV) {
        if (w.part > 0) {
            float *xc = o.xcarry + wave_slot * kHalo * kLanes + w.lane;
#pragma unroll
            for (int j = 0; j < kHalo; ++j)
                xc[j * kLanes] = acc.ring[j];
        }
    }
    if (w.active) {
        const int64_t slot = c.b * parts + w.part;
#pragma unroll
        for (int n = 0; n < N; ++n)
            o.pA[(slot * dim + w.d) * N + n] = dA[n];
        o.pD[slot * dim + w.d] = acc.dD;
        o.pbias[slot * dim + w.d] = acc.dbias;
        if constexpr (CONV) {
            // tap m of the zero-padded window is conv_weight[d, m - (4 - conv_k)]
            const int k = ext.conv_k;
#pragma unroll
            for (int m = 0; m < kMaxConv; ++m)
                if (m >= kMaxConv - k)
                    o.pW[(slot * dim + w.d) * k + m - (kMaxConv - k)] = acc.dcw[m];
            o.pWb[slot * dim + w.d] = acc.dcb;
        }
        if (w.part == 0 && o.dh0) {
#pragma unroll
            for (int n = 0; n < N; ++n)
                o.dh0[(c.b * dim + w.d) * N + n] = g[n];
        }
    }
}

// Conv prologue: dx of the last kHalo steps of every part but the last, the
// part's own share plus the next part's.
template <typename TIO>
__global__ __launch_bounds__(kLanes * 4) void bwd_conv_fixup_kernel(
    TIO *__restrict__ du, const float *__restrict__ xown, const float *__restrict__ xcarry,
    int64_t L, int64_t dim, int64_t groups, int parts, int64_t part_len, int rev)
{
    WaveSetup w;
    const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (!setup_wave(w, gw, groups, parts - 1, L, dim, part_len, (int)sizeof(TIO), rev))
        return;
    const WaveCtx &c = w.c;
    const int64_t slot = w.grp * parts + w.part;
#pragma unroll
    for (int j = 0; j < kHalo; ++j) {
        const float v = xown[(slot * kHalo + j) * kLanes + w.lane] +
                        xcarry[((slot + 1) * kHalo + j) * kLanes + w.lane];
        const int64_t s = c.l_end - 1 - j;
        if (w.active)
            store_elem(du, scan_row<kVarExt>(c, s) * dim + w.d, v);
    }
}

// ---------------------------------------------------------------------------
// 5. reductions of the partials (fixed order), workspace layout and launch
// ---------------------------------------------------------------------------
// Column sums of the partials (bwd_stream.hip): every reduction of one call
// in one launch.
constexpr int kMaxColsumJobs = 7;
struct ColsumJob {
    const float *in;
    float *out;
    int64_t P, K, block0;
};
struct ColsumJobs {
    ColsumJob j[kMaxColsumJobs] = {};
    int n = 0;
    int64_t blocks = 0;
    void add(const float *in, float *out, int64_t P, int64_t K);
};
hipError_t launch_colsums(const ColsumJobs &jobs, hipStream_t s);

struct BwdLayout {
    StreamPlan p;
    int64_t nck, gpr;
    size_t fsumm, asumm, fentry, aentry, carry, ckpt, pB, pC, pA, pD, pbias, pW, pWb, xown,
        xcarry, total;   // byte offsets
};
BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t dim, int64_t N);

template <int N, int VAR, typename TIO>
hipError_t launch_bwd_n(const BwdArgs &a, const FwdExt &e, hipStream_t s)
{
    constexpr bool CONV = (VAR & kVarConv) != 0;
    const BwdLayout w = bwd_layout(a.fwd.batch, a.fwd.L, a.fwd.dim, N);
    char *base = (char *)(((uintptr_t)a.fwd.workspace + 255) & ~(uintptr_t)255);
    float *fsumm = (float *)(base + w.fsumm), *asumm = (float *)(base + w.asumm);
    float *fentry = (float *)(base + w.fentry), *aentry = (float *)(base + w.aentry);
    float *ckpt = (float *)(base + w.ckpt);
    BwdOut o;
    o.du = a.du; o.ddelta = a.ddelta; o.dz = a.dz;
    o.pB = (float *)(base + w.pB); o.pC = (float *)(base + w.pC);
    o.pA = (float *)(base + w.pA); o.pD = (float *)(base + w.pD);
    o.pbias = (float *)(base + w.pbias);
    o.dh0 = a.dh0;
    o.pW = (float *)(base + w.pW); o.pWb = (float *)(base + w.pWb);
    o.xown = (float *)(base + w.xown); o.xcarry = (float *)(base + w.xcarry);
    ExtParams x;
    x.conv_w = CONV ? e.conv_w : nullptr;
    x.conv_b = CONV ? e.conv_b : nullptr;
    x.conv_k = CONV ? e.conv_k : 0;
    x.rev = (e.flags & kFwdFlagReverse) ? 1 : 0;
    // VAR = 0: Euler B_bar, forward direction, addressing fixed at compile time
    constexpr bool plain = VAR == 0;
    const StreamPlan &p = w.p;
    hipError_t err;
    const bool split = p.parts > 1;
    float *cscr = (float *)(base + w.carry);   // shared: the two carries run in turn
    // With the forward's part state reused, its summaries are in place, and
    // its entry states too unless it folded the summaries in its main pass
    // (a few parts: no carry launch, no entry states written).
    const bool reuse = (e.flags & kBwdFlagReuseFwdState) != 0;
    const bool have_fentry = reuse && p.parts > stream::kFoldInKernelMaxParts;
    if (split && !reuse) {
        err = plain ? launch_fwd_summaries(a.fwd, p, fsumm, s)
                    : launch_fwd_summaries_ext(a.fwd, e, p, fsumm, s);
        if (err != hipSuccess)
            return err;
    }
    const int64_t adj_blocks = split ? (p.groups * (p.parts - 1) + 3) / 4 : 0;
    const int64_t ck_blocks = (p.groups * p.parts + 3) / 4;
    auto pass23 = [&](auto kernel, int64_t nadj, int64_t nck) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)(nadj + nck)), dim3(kLanes * 4), 0, s,
                           (const TIO *)a.fwd.u, (const TIO *)a.fwd.delta, (const TIO *)a.fwd.z,
                           (const TIO *)a.dy, a.fwd.A, (const TIO *)a.fwd.Bm,
                           (const TIO *)a.fwd.Cm, a.fwd.delta_bias, a.fwd.delta_softplus,
                           a.fwd.h0, (const float *)(split ? fentry : nullptr), asumm, ckpt, w.nck,
                           x, a.fwd.L, a.fwd.dim, p.groups, p.parts, p.part_len, nadj, nck);
    };
    // entry states of the parts: from the left (h0) and from the right (dh_last)
    auto carry_fwd = [&]() {
        return split && !have_fentry
                   ? launch_fwd_carry(fsumm, a.fwd.h0, a.fwd.A, fentry, a.fwd.batch, a.fwd.dim,
                                      N, p.parts, 0, cscr, s)
                   : hipSuccess;
    };
    auto carry_adj = [&]() {
        return split ? launch_fwd_carry(asumm, a.dh_last, a.fwd.A, aentry, a.fwd.batch,
                                        a.fwd.dim, N, p.parts, 1, cscr, s)
                     : hipSuccess;
    };
    if constexpr ((VAR & kVarZoh) == 0) {
        // the checkpoints need the forward entry states
        if ((err = carry_fwd()) != hipSuccess)
            return err;
        pass23(bwd_pass23_kernel<N, VAR, 3, TIO>, adj_blocks, ck_blocks);
        if ((err = hipGetLastError()) != hipSuccess || (err = carry_adj()) != hipSuccess)
            return err;
    } else {
        // checkpoints last, just before the main pass that reads them
        if (adj_blocks > 0)
            pass23(bwd_pass23_kernel<N, VAR, 1, TIO>, adj_blocks, 0);
        if ((err = hipGetLastError()) != hipSuccess || (err = carry_fwd()) != hipSuccess ||
            (err = carry_adj()) != hipSuccess)
            return err;
        pass23(bwd_pass23_kernel<N, VAR, 2, TIO>, 0, ck_blocks);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    const int64_t waves = p.groups * p.parts;
    hipLaunchKernelGGL((bwd_main_kernel<N, VAR, TIO>), dim3((unsigned)waves), dim3(kLanes), 0, s,
                       (const TIO *)a.fwd.u, (const TIO *)a.fwd.delta, (const TIO *)a.fwd.z,
                       (const TIO *)a.dy, a.fwd.A, (const TIO *)a.fwd.Bm, (const TIO *)a.fwd.Cm,
                       a.fwd.D_skip, a.fwd.delta_bias, a.fwd.delta_softplus, a.dh_last,
                       (const float *)(split ? aentry : nullptr), ckpt, o, a.fwd.L, a.fwd.dim,
                       a.fwd.batch, p.groups, p.parts, p.part_len, w.nck, x);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    if (CONV && p.parts > 1) {
        const int64_t fw = p.groups * (p.parts - 1);
        hipLaunchKernelGGL((bwd_conv_fixup_kernel<TIO>), dim3((unsigned)((fw + 3) / 4)),
                           dim3(kLanes * 4), 0, s, (TIO *)a.du, (const float *)o.xown,
                           (const float *)o.xcarry, a.fwd.L, a.fwd.dim, p.groups, p.parts,
                           p.part_len, x.rev);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    const int64_t count = a.fwd.batch * a.fwd.L * N;
    const int64_t slots = a.fwd.batch * p.parts;
    ColsumJobs jobs;
    jobs.add(o.pB, a.dB, count, w.gpr);
    jobs.add(o.pC, a.dC, count, w.gpr);
    jobs.add(o.pA, a.dA, a.fwd.dim * N, slots);
    jobs.add(o.pD, a.dD, a.fwd.dim, slots);
    jobs.add(o.pbias, a.ddelta_bias, a.fwd.dim, slots);
    if (CONV) {
        jobs.add(o.pW, a.dconv_w, a.fwd.dim * x.conv_k, slots);
        jobs.add(o.pWb, a.dconv_b, a.fwd.dim, slots);
    }
    return launch_colsums(jobs, s);
}

template <int VAR>
hipError_t launch_bwd_var(const BwdArgs &a, const FwdExt &e, hipStream_t s)
{
#define SELSCAN_BWD_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return a.fwd.dtype == 1 ? launch_bwd_n<NN, VAR, uint16_t>(a, e, s)                        \
                                : launch_bwd_n<NN, VAR, float>(a, e, s);
    switch (a.fwd.N) {
    SELSCAN_BWD_CASE(4)
    SELSCAN_BWD_CASE(8)
    SELSCAN_BWD_CASE(16)
    SELSCAN_BWD_CASE(32)
    SELSCAN_BWD_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_BWD_CASE
}

} // namespace bwd
} // namespace selscan
