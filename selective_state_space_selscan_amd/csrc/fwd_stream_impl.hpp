// Streaming selective-scan forward for gfx950: kernel templates shared by the
// default instantiation (fwd_stream.hip) and the variant instantiations
// (fwd_stream_ext_n*.hip).
//
// What it computes is the S6 recurrence of the Mamba tutorial (pwwt.cn)
// §3.1-§3.2 and §4.2: Delta_t = softplus(Delta_raw + bias), A_bar = exp(Delta_t A)
// with diagonal A, h_t = A_bar_t h_{t-1} + Delta_t B_t u_t, y_t = C_t.h_t + D u_t,
// times SiLU(z_t).  Discretisation, recurrence and readout run fused in one
// kernel with the state in registers (tutorial §3.2, Gu & Dao deep-reading
// report §2.4); only y (and h_L if asked) reaches HBM.
//
// Work decomposition: every wavefront is independent (no barriers, no LDS).
//   * lane = one channel d of a 64-channel group of one batch row, so the
//     u/Delta/z/y accesses of a wave are one contiguous row per timestep and
//     B_t, C_t are wave-uniform: scalar loads into SGPRs, used directly as
//     VALU operands.
//   * wave = one (channel group, sequence part).  It walks its part of the
//     sequence step by step with the N-entry state of each lane in VGPRs:
//     per (t, n) one multiply for A_bar (see below), one for Delta B u, one FMA
//     for the state and one FMA for the readout.
//   * inputs of the next TT steps are loaded while the current TT are
//     computed (two register buffers, no branch between them).
// The sequence is split into P parts so that batch * dim / 64 * P waves fill
// the chip.  A summary pass (SUMMARY = true) runs each part but the last from
// a zero state and stores (sum of Delta over the part, end state); h0 is then
// folded through the summaries of parts 0..p-1 with the associative operator
// (a, b) o (c, d) = (a c, a d + b) of the selection-mechanism article
// (discosf.com) §3.1, where the decay of a whole part is exp(A sum Delta): for
// a carry kernel (fwd_stream.hip) that stores the entry state of every part,
// read once by the main pass, or for a few parts (kFoldInKernelMaxParts) by
// each main-pass wave itself, which saves the carry launch.
//
// Structured A: when every A[d, n] equals (n+1) A[d, 0] exactly (the S4D-real
// initialisation A = -exp(log(1..N)) of the tutorial's §4.2 listing),
// exp(Delta A[d, n]) = r^(n+1) with r = exp(Delta A[d, 0]), one multiply per
// (t, n) instead of a multiply and an exp2.  A wave uses it only if all its
// channels qualify; any other A takes the exp2 path.
//
// Variants (VAR has kVarExt set; the default instantiation VAR = 0 compiles
// none of this):
//   * reverse direction (runtime flag): the scan runs over the time-reversed
//     sequence, t = L-1 down to 0 (the bidirectional use named in the
//     tutorial's §7 outlook).  Parts, summaries and the fold are unchanged in
//     scan order; only the scalar addressing maps scan step s to t = L-1-s.
//   * exact zero-order hold (kVarZoh): B_bar = (exp(Delta A) - 1) / A * B
//     (tutorial §2.2; selection-mechanism article §2.1) in place of Delta B.
//   * causal depthwise conv1d + SiLU prologue (kVarConv): the scan input is
//     u_s = SiLU(conv_bias + sum_j w_j x_{s-k+1+j}) over the raw input x, with
//     x = 0 before the first step (tutorial §3.3 and its §4.2 listing: a
//     grouped Conv1d with padding k-1 cut to the first L outputs, then SiLU).
//     The last k-1 inputs ride along in registers.
#pragma once

#include "buffer_io.hpp"
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {
namespace stream {

constexpr int kLanes = 64;
constexpr int kWavesPerBlock = 4;
constexpr int TT = 4;   // timesteps per prefetch buffer, main pass
constexpr int TTS = 8;  // timesteps per prefetch buffer, summary pass
// A store offset past the byte range of every output descriptor (a chunk's
// range is at most TT * dim * 4 bytes, and dim * 4 < 2^26 is checked on the
// host), so stores from lanes past dim are dropped by the hardware.
constexpr int kStoreOffsetOutOfRange = 1 << 30;
static_assert(TT <= kStreamTT, "plan rounds parts to kStreamTT steps");

// kVarRev: reverse direction fixed at compile time, used alone (no kVarExt):
// the reverse-only call then compiles to the default's code with the
// addressing mirrored.  kVarUf (backward only): the scan input is fp32 bits
// whatever the I/O type (the conv prologue's output, computed beforehand).
// kVarKeep (the main pass of the default forward, alone or with kVarRev):
// the pass also stores the state entering every TT-step chunk (in scan
// order), the checkpoints a backward that reuses this forward's workspace
// would otherwise recompute.
enum : int { kVarExt = 1, kVarZoh = 2, kVarConv = 4, kVarRev = 8, kVarUf = 16, kVarKeep = 32 };
constexpr int kMaxConv = 4;

// Variant arguments of the kernel (ignored when VAR = 0).
struct ExtParams {
    const float *conv_w;   // (dim, conv_k), or null
    const float *conv_b;   // (dim), or null
    int conv_k;
    int rev;
    float *ckpt;           // kVarKeep: (groups, nck, N, 64) states entering each chunk
    int64_t nck;           // chunks per channel group: ceil(L / TT)
};

template <int TTc>
struct ChunkT {
    uint32_t u[TTc], x[TTc], z[TTc];   // raw element bits, widened at use
};
using Chunk = ChunkT<TT>;

struct WaveCtx {
    int64_t b, d0, L, dim, l_begin, l_end;   // l_begin, l_end: part, in scan steps
    int64_t bL;        // b * L: row of timestep 0 of this batch row
    int voff, row_bytes;
    int voff_store;    // voff, or an offset past every descriptor range for lanes past dim
    float bias, Dd, A2_0;
    int rev;           // variants: 1 = scan step s is timestep L-1-s
    int softplus;      // variants: Delta = softplus(Delta_raw + bias) (else the sum)
    float invA0;       // exact ZOH: 1 / A[d, 0]
    float cw[kMaxConv], cb;   // conv prologue: taps (zero-padded in front), bias
};

// Row b*L + t of the (batch, L, .) arrays for scan step s.
template <int VAR>
__device__ __forceinline__ int64_t scan_row(const WaveCtx &c, int64_t s)
{
    if constexpr ((VAR & kVarRev) != 0)
        return c.bL + c.L - 1 - s;
    else if constexpr ((VAR & kVarExt) != 0)
        return c.bL + (c.rev ? c.L - 1 - s : s);
    else
        return c.bL + s;
}

// Row step between consecutive scan steps: +1, or -1 in reverse direction.
template <int VAR>
__device__ __forceinline__ int64_t row_dir(const WaveCtx &c)
{
    if constexpr ((VAR & kVarRev) != 0)
        return -1;
    else if constexpr ((VAR & kVarExt) != 0)
        return c.rev ? -1 : 1;
    else
        return 1;
}

// A run of `rows` consecutive scan steps starting at s0 occupies the
// timesteps [t_lo, t_lo + rows).  Step i of the run sits at scalar offset
// step_soff(...) from the element (t_lo, d0); steps at or past `rows` get an
// offset past the descriptor range (reverse direction), or lie past it anyway.
template <int VAR>
__device__ __forceinline__ int64_t run_t_lo(const WaveCtx &c, int64_t s0, int64_t rows)
{
    if constexpr ((VAR & kVarRev) != 0)
        return c.L - s0 - rows;
    else if constexpr ((VAR & kVarExt) != 0)
        return c.rev ? c.L - s0 - rows : s0;
    else
        return s0;
}
template <int VAR>
__device__ __forceinline__ int step_soff(const WaveCtx &c, int i, int rows)
{
    if constexpr ((VAR & kVarRev) != 0) {
        return i < rows ? (rows - 1 - i) * c.row_bytes : kStoreOffsetOutOfRange;
    } else if constexpr ((VAR & kVarExt) != 0) {
        if (c.rev)
            return i < rows ? (rows - 1 - i) * c.row_bytes : kStoreOffsetOutOfRange;
    }
    return i * c.row_bytes;
}

// Raw dwords of one B_t or C_t row (N values, two bf16 or one fp32 per dword).
template <int N, typename TIO>
struct RowRaw {
    static constexpr int W = N * (int)sizeof(TIO) / 4;
    uint32_t w[W];
};

template <int N, typename TIO>
__device__ __forceinline__ void fetch_row(RowRaw<N, TIO> &r, const TIO *p, int64_t row)
{
    const const_u32 *q = as_const_u32(p) + row * RowRaw<N, TIO>::W;
#pragma unroll
    for (int k = 0; k < RowRaw<N, TIO>::W; ++k)
        r.w[k] = q[k];
}

template <int N>
__device__ __forceinline__ float row_val(const RowRaw<N, float> &r, int n)
{
    return __uint_as_float(r.w[n]);
}
template <int N>
__device__ __forceinline__ float row_val(const RowRaw<N, uint16_t> &r, int n)
{
    const uint32_t w = r.w[n >> 1];
    return __uint_as_float((n & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <bool GATED, int VAR, int TTc, typename TIO>
__device__ __forceinline__ void load_chunk(ChunkT<TTc> &ch, const TIO *u, const TIO *delta,
                                           const TIO *z, const WaveCtx &c, int64_t t0)
{
    constexpr int TT = TTc;
    int64_t rows = c.l_end - t0;
    rows = rows < 0 ? 0 : (rows > TT ? TT : rows);
    if (t0 < c.l_begin)
        rows = 0;
    const int64_t elem = (c.bL + run_t_lo<VAR>(c, t0, rows)) * c.dim + c.d0;
    // A chunk outside the part has an empty range: its loads return 0 and
    // read nothing (the prefetch runs one chunk past either end).
    const int64_t bytes = rows > 0 ? (rows * c.dim - c.d0) * (int64_t)sizeof(TIO) : 0;
    const int64_t safe_elem = rows > 0 ? elem : 0;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + safe_elem, bytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + safe_elem, bytes);
#pragma unroll
    for (int i = 0; i < TT; ++i)
        ch.x[i] = buf_load_raw(rd, c.voff, step_soff<VAR>(c, i, (int)rows), delta);
#pragma unroll
    for (int i = 0; i < TT; ++i)
        ch.u[i] = buf_load_raw(ru, c.voff, step_soff<VAR>(c, i, (int)rows), u);
    if (GATED) {
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + safe_elem, bytes);
#pragma unroll
        for (int i = 0; i < TT; ++i)
            ch.z[i] = buf_load_raw(rz, c.voff, step_soff<VAR>(c, i, (int)rows), z);
    }
}

// Scan input of one step: the loaded value, or with the conv prologue the
// causal conv over the last kMaxConv raw inputs, then SiLU.  win holds the
// kMaxConv - 1 raw inputs before this step, oldest first.
template <int VAR, typename TIO>
__device__ __forceinline__ float step_input(uint32_t raw, const WaveCtx &c,
                                            float (&win)[kMaxConv - 1])
{
    const float x = (VAR & kVarUf) != 0 ? __uint_as_float(raw) : raw_to_f32(raw, tag<TIO>());
    if constexpr ((VAR & kVarConv) != 0) {
        float acc = c.cb;
#pragma unroll
        for (int j = 0; j < kMaxConv - 1; ++j)
            acc = fmaf(c.cw[j], win[j], acc);
        acc = fmaf(c.cw[kMaxConv - 1], x, acc);
#pragma unroll
        for (int j = 0; j < kMaxConv - 2; ++j)
            win[j] = win[j + 1];
        win[kMaxConv - 2] = x;
        return silu(acc);
    } else {
        return x;
    }
}

// Delta of one step.  The default instantiation has the softplus switch as a
// template argument; the variants select at run time (one instantiation less).
template <bool SOFTPLUS, int VAR>
__device__ __forceinline__ float step_delta(float x, const WaveCtx &c)
{
    if constexpr ((VAR & kVarExt) != 0) {
        const float sp = softplus(x);
        return c.softplus ? sp : x;
    } else {
        return SOFTPLUS ? softplus(x) : x;
    }
}

// Exact zero-order-hold coefficient (exp(Delta a) - 1) / a, given
// x2 = Delta a log2(e) and e = 2^x2 = exp(Delta a).  Where |Delta a| is
// small, e - 1 cancels, so the Taylor series of Delta * (e^x - 1) / x in
// x = Delta a (degree 4, truncation below 1e-8 relative for |x2| < 1/8) is
// used there; elsewhere the cancellation costs at most 1 ulp(e) / |e - 1|,
// below 1e-6 relative.  a = 0 gives x2 = 0 and the series value Delta.
__device__ __forceinline__ float zoh_coeff(float dt, float x2, float e, float inv_a)
{
    constexpr float k1 = kLn2 / 2.0f;
    constexpr float k2 = kLn2 * kLn2 / 6.0f;
    constexpr float k3 = kLn2 * kLn2 * kLn2 / 24.0f;
    constexpr float k4 = kLn2 * kLn2 * kLn2 * kLn2 / 120.0f;
    const float series = dt * fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, k4, k3), k2), k1), 1.0f);
    const float direct = (e - 1.0f) * inv_a;
    return fabsf(x2) < 0.125f ? series : direct;
}

// TT steps of the recurrence on one prefetched chunk.  FULL: all TT steps are
// inside the range (no per-step check); otherwise steps past the end are the
// identity element (Delta = 0).  The B_t / C_t rows of step i+1 are fetched
// (scalar loads) while step i computes.  The loop body has no branch, so the
// scheduler is free to move loads ahead.
template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, bool FULL, int VAR,
          typename TIO>
__device__ __forceinline__ void run_chunk(const Chunk &ch, const TIO *Bm, const TIO *Cm, TIO *y,
                                          const WaveCtx &c, int64_t t0, const float (&A2)[N],
                                          const float (&invA)[N], float (&h)[N], float &sdelta,
                                          float (&win)[kMaxConv - 1])
{
    constexpr bool ZOH = (VAR & kVarZoh) != 0;
    const int rows = FULL ? TT : (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    const int64_t elem = (c.bL + run_t_lo<VAR>(c, t0, rows)) * c.dim + c.d0;
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(SUMMARY ? nullptr : y + elem, SUMMARY ? 0 : (rows * c.dim - c.d0) * (int64_t)sizeof(TIO));
    const int64_t row0 = scan_row<VAR>(c, t0);
    const int64_t row_last = scan_row<VAR>(c, c.L - 1);
    const int64_t dir = row_dir<VAR>(c);
    RowRaw<N, TIO> bcur, ccur, bnxt, cnxt;
    fetch_row(bcur, Bm, row0);
    if (!SUMMARY)
        fetch_row(ccur, Cm, row0);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        if (i + 1 < TT) {
            // steps past L read the last row (padding steps, never stored)
            const int64_t rn = (FULL || t0 + i + 1 <= c.L - 1) ? row0 + (i + 1) * dir : row_last;
            fetch_row(bnxt, Bm, rn);
            if (!SUMMARY)
                fetch_row(cnxt, Cm, rn);
        }
        const bool valid = FULL || i < rows;
        const float ut = step_input<VAR, TIO>(ch.u[i], c, win);
        const float x = raw_to_f32(ch.x[i], tag<TIO>()) + c.bias;
        float dt = step_delta<SOFTPLUS, VAR>(x, c);
        if (!FULL)
            dt = valid ? dt : 0.0f;        // padding steps are the identity (1, 0)
        const float du = dt * ut;
        float yv = c.Dd * ut;
        const float r = POW ? exp2_decay(dt * c.A2_0, tag<TIO>()) : 0.0f;
        float pw = 1.0f;
        // exact ZOH with structured A: r^(n+1) - 1 = (r - 1)(1 + r + ... + r^n),
        // so B_bar_n / B_n = em * S_n / (n+1) with em = (r - 1) / A[d,0] and
        // S_n = 1 + r + ... + r^n (a running sum of the powers).
        const float g = (ZOH && POW) ? zoh_coeff(dt, dt * c.A2_0, r, c.invA0) * ut : 0.0f;
        float S = 1.0f;
        if (SUMMARY)
            sdelta += dt;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            float a, bu;
            if constexpr (ZOH) {
                if (POW) {
                    a = (pw *= r);
                    bu = (g * (1.0f / (float)(n + 1))) * (S * row_val<N>(bcur, n));
                    S += a;
                } else {
                    const float x2 = dt * A2[n];
                    a = exp2_decay(x2, tag<TIO>());
                    bu = zoh_coeff(dt, x2, a, invA[n]) * (ut * row_val<N>(bcur, n));
                }
            } else {
                a = POW ? (pw *= r) : exp2_decay(dt * A2[n], tag<TIO>());
                bu = du * row_val<N>(bcur, n);
            }
            h[n] = fmaf(a, h[n], bu);
            if (!SUMMARY)
                yv = fmaf(row_val<N>(ccur, n), h[n], yv);
        }
        if (!SUMMARY) {
            if (GATED)
                yv *= silu(raw_to_f32(ch.z[i], tag<TIO>()));
            // rows past the end and lanes past dim fall outside the descriptor
            buf_store(ry, c.voff_store, step_soff<VAR>(c, i, rows), yv, y);
        }
        if (i + 1 < TT) {
            bcur = bnxt;
            if (!SUMMARY)
                ccur = cnxt;
        }
    }
}

template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, int VAR, typename TIO>
__device__ __forceinline__ void run_any_chunk(const Chunk &ch, const TIO *Bm, const TIO *Cm, TIO *y,
                                              const WaveCtx &c, int64_t t0,
                                              const float (&A2)[N], const float (&invA)[N],
                                              float (&h)[N], float &sdelta,
                                              float (&win)[kMaxConv - 1])
{
    if (t0 + TT <= c.l_end)
        run_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, true, VAR>(ch, Bm, Cm, y, c, t0, A2, invA, h,
                                                               sdelta, win);
    else
        run_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, false, VAR>(ch, Bm, Cm, y, c, t0, A2, invA, h,
                                                                sdelta, win);
}

// Forward walk over the part (main pass, and the summary for general A).
// kVarKeep: ck is this wave's lane of its channel group's checkpoints, and
// the state entering each chunk is stored there first (every lane, those past
// dim too: their values are finite and a reader may combine them with zeros).
template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, int VAR, typename TIO>
__device__ __forceinline__ void run_part(const TIO *u, const TIO *delta, const TIO *z, TIO *y,
                                         const TIO *Bm, const TIO *Cm, const WaveCtx &c,
                                         const float (&A2)[N], const float (&invA)[N],
                                         float (&h)[N], float &sdelta, float (&win)[kMaxConv - 1],
                                         float *ck = nullptr)
{
    auto keep = [&](int64_t t) {
        if constexpr ((VAR & kVarKeep) != 0 && !SUMMARY) {
#pragma unroll
            for (int n = 0; n < N; ++n)
                ck[(t / TT) * (N * kLanes) + n * kLanes] = h[n];
        }
    };
    Chunk A, B;
    int64_t t0 = c.l_begin;
    load_chunk<GATED, VAR>(A, u, delta, z, c, t0);
    for (;;) {
        load_chunk<GATED, VAR>(B, u, delta, z, c, t0 + TT);
        keep(t0);
        run_any_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, VAR>(A, Bm, Cm, y, c, t0, A2, invA, h,
                                                             sdelta, win);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
        load_chunk<GATED, VAR>(A, u, delta, z, c, t0 + TT);
        keep(t0);
        run_any_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, VAR>(B, Bm, Cm, y, c, t0, A2, invA, h,
                                                             sdelta, win);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
    }
}

// Summary of a part for structured A, walking the part backwards in time.
// The end state from zero is x[n] = sum_t Q_t^(n+1) Delta_t u_t B_t[n], with
// Q_t = prod_{s>t} r_s and r_s = exp(Delta_s A[d,0]).  Walking backwards, Q
// is one running product and Delta_t u_t Q_t^(n+1) one multiply per n, so a
// (t, n) costs a multiply and an FMA (the forward walk needs three ops);
// with exact ZOH three operations (the forward walk: six).  With the
// conv prologue the input of step i needs the raw inputs of steps i-3..i:
// inside the chunk, or for its first steps the last raw inputs of the chunk
// before it (prev: the next chunk of the walk, prefetched while this one
// computes, and needed only at the end of this one's walk) or, at the start
// of the part, the window before the part (win).
template <int N, bool SOFTPLUS, bool FULL, int VAR, typename TIO>
__device__ __forceinline__ void summary_chunk_rev(const ChunkT<TTS> &ch, const ChunkT<TTS> &prev,
                                                  bool prev_in_part,
                                                  const float (&win)[kMaxConv - 1],
                                                  const TIO *Bm, const WaveCtx &c, int64_t t0,
                                                  float &Q, float (&x)[N], float &sdelta)
{
    constexpr int TT = TTS;
    constexpr bool CONV = (VAR & kVarConv) != 0;
    static_assert(TT >= kMaxConv - 1, "the conv window reaches one chunk back at most");
    // raw input of chunk step j, j >= -(kMaxConv - 1)
    auto raw_in = [&](int j) -> float {
        if (j >= 0)
            return raw_to_f32(ch.u[j], tag<TIO>());
        return prev_in_part ? raw_to_f32(prev.u[TT + j], tag<TIO>()) : win[kMaxConv - 1 + j];
    };
    const int rows = FULL ? TT : (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    // B_t row of step i-1 is fetched (scalar loads) while step i computes.
    const int64_t row0 = scan_row<VAR>(c, t0);
    const int64_t dir = row_dir<VAR>(c);
    RowRaw<N, TIO> bcur, bnxt;
    fetch_row(bcur, Bm, row0 + (FULL ? TT - 1 : rows - 1) * dir);
#pragma unroll
    for (int i = TT - 1; i >= 0; --i) {
        if (!FULL && i >= rows)
            continue;   // uniform: steps past the end contribute nothing
        if (i > 0)
            fetch_row(bnxt, Bm, row0 + (i - 1) * dir);
        float ut;
        if constexpr (CONV) {
            // the main pass's step_input: the same FMAs in the same order
            float acc = c.cb;
#pragma unroll
            for (int m = 0; m < kMaxConv; ++m)
                acc = fmaf(c.cw[m], raw_in(i - (kMaxConv - 1) + m), acc);
            ut = silu(acc);
        } else {
            ut = raw_to_f32(ch.u[i], tag<TIO>());
        }
        const float xr = raw_to_f32(ch.x[i], tag<TIO>()) + c.bias;
        const float dt = step_delta<SOFTPLUS, VAR>(xr, c);
        sdelta += dt;
        const float r = exp2_decay(dt * c.A2_0, tag<TIO>());
        if constexpr ((VAR & kVarZoh) != 0) {
            // Exact ZOH: the step adds Q^(n+1) g S_n / (n+1) B_t[n], with
            // g = (r - 1) / A[d,0] * u and S_n = 1 + r + ... + r^n.  P_n =
            // Q^(n+1) S_n g follows P_n = Q P_(n-1) + T_n, T_n = Q^(n+1) r^n g =
            // T_(n-1) Q r; the 1/(n+1) is applied once at the end of the part
            // (summary_part_rev): three operations per (t, n).
            const float qr = Q * r;
            float T = zoh_coeff(dt, dt * c.A2_0, r, c.invA0) * ut * Q;
            float P = T;
            x[0] = fmaf(P, row_val<N>(bcur, 0), x[0]);
#pragma unroll
            for (int n = 1; n < N; ++n) {
                T *= qr;
                P = fmaf(Q, P, T);
                x[n] = fmaf(P, row_val<N>(bcur, n), x[n]);
            }
        } else {
            float g = dt * ut * Q;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                if (n)
                    g *= Q;
                x[n] = fmaf(g, row_val<N>(bcur, n), x[n]);
            }
        }
        Q *= r;
        if (i > 0)
            bcur = bnxt;
    }
}

template <int N, bool SOFTPLUS, int VAR, typename TIO>
__device__ __forceinline__ void summary_part_rev(const TIO *u, const TIO *delta, const TIO *Bm,
                                                 const WaveCtx &c,
                                                 const float (&win)[kMaxConv - 1],
                                                 float (&x)[N], float &sdelta)
{
    constexpr int TT = TTS;
    const int64_t nchunks = (c.l_end - c.l_begin + TT - 1) / TT;
    ChunkT<TTS> A, B;
    float Q = 1.0f;
    int64_t k = nchunks - 1;
    int64_t t0 = c.l_begin + k * TT;
    load_chunk<false, VAR>(A, u, delta, (const TIO *)nullptr, c, t0);
    // the last chunk may be partial; every other chunk is full
    load_chunk<false, VAR>(B, u, delta, (const TIO *)nullptr, c, t0 - TT);
    if (t0 + TT <= c.l_end)
        summary_chunk_rev<N, SOFTPLUS, true, VAR>(A, B, k > 0, win, Bm, c, t0, Q, x, sdelta);
    else
        summary_chunk_rev<N, SOFTPLUS, false, VAR>(A, B, k > 0, win, Bm, c, t0, Q, x, sdelta);
    for (;;) {
        if (--k < 0)
            break;
        t0 -= TT;
        load_chunk<false, VAR>(A, u, delta, (const TIO *)nullptr, c, t0 - TT);
        summary_chunk_rev<N, SOFTPLUS, true, VAR>(B, A, k > 0, win, Bm, c, t0, Q, x, sdelta);
        if (--k < 0)
            break;
        t0 -= TT;
        load_chunk<false, VAR>(B, u, delta, (const TIO *)nullptr, c, t0 - TT);
        summary_chunk_rev<N, SOFTPLUS, true, VAR>(A, B, k > 0, win, Bm, c, t0, Q, x, sdelta);
    }
    if constexpr ((VAR & kVarZoh) != 0) {
#pragma unroll
        for (int n = 1; n < N; ++n)
            x[n] *= 1.0f / (float)(n + 1);
    }
}

// Conv prologue taps of channel d, aligned to the newest input (zeros in
// front when conv_k < kMaxConv), and the conv bias.
__device__ __forceinline__ void conv_taps(WaveCtx &c, const ExtParams &ext, int64_t d)
{
#pragma unroll
    for (int m = 0; m < kMaxConv; ++m) {
        const int j = m - (kMaxConv - ext.conv_k);
        c.cw[m] = j >= 0 ? ext.conv_w[d * ext.conv_k + j] : 0.0f;
    }
    c.cb = ext.conv_b ? ext.conv_b[d] : 0.0f;
}

// Raw inputs of the kMaxConv - 1 scan steps before the part, oldest first
// (zero before scan step 0).
template <int VAR, typename TIO>
__device__ __forceinline__ void conv_window(float (&win)[kMaxConv - 1], const WaveCtx &c,
                                            const TIO *u, int64_t d)
{
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j) {
        const int64_t s = c.l_begin - (kMaxConv - 1) + j;
        win[j] = s >= 0 ? load_elem(u, scan_row<VAR>(c, s) * c.dim + d) : 0.0f;
    }
}

// Entry state of a part: entry[(grp * parts + part) * N + n][lane] (written by
// the carry kernel from the part summaries), one coalesced row per n.
template <int N>
__device__ __forceinline__ void load_entry(float (&h)[N], const float *entry, int64_t grp,
                                           int parts, int part, int lane)
{
    const float *e = entry + ((grp * parts + part) * (int64_t)N) * kLanes + lane;
#pragma unroll
    for (int n = 0; n < N; ++n)
        h[n] = e[n * kLanes];
}

// h <- exp(A S) h + x for one part summary v = (S, x[0..N-1]); for structured
// A, exp(A[d,n] S) = e^(n+1) with e = exp(A[d,0] S).
constexpr int kFoldGroup = 4;
// Up to this many parts the main pass folds the summaries itself (each wave
// at most kFoldInKernelMaxParts - 1 of them) instead of reading entry states
// from a carry launch.
constexpr int kFoldInKernelMaxParts = 4;
template <int N>
__device__ __forceinline__ void fold_part_summary(float (&h)[N], const float (&v)[N + 1],
                                                  bool pow_path, const float (&A2)[N],
                                                  float A2_0)
{
    const float S = v[0];
    if (pow_path) {
        const float e = hw_exp2(A2_0 * S);
        float pw = 1.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            pw *= e;
            h[n] = fmaf(pw, h[n], v[n + 1]);
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = fmaf(hw_exp2(A2[n] * S), h[n], v[n + 1]);
    }
}

// Folds `count` part summaries into h, the summary indices first, first + dir,
// ...  sbase points at summary 0 of this lane's channel group (summaries are
// (N + 1) * 64 floats apart).  The summaries are read kFoldGroup at a time,
// all loads first, so a wave waits for memory once per group rather than
// once per part.
template <int N>
__device__ __forceinline__ void fold_summaries(float (&h)[N], const float *sbase, int first,
                                               int count, int dir, bool pow_path,
                                               const float (&A2)[N], float A2_0)
{
    int k0 = 0;
    for (; k0 + kFoldGroup <= count; k0 += kFoldGroup) {
        float v[kFoldGroup][N + 1];
#pragma unroll
        for (int k = 0; k < kFoldGroup; ++k) {
            const float *s = sbase + (int64_t)(first + (k0 + k) * dir) * (N + 1) * kLanes;
#pragma unroll
            for (int n = 0; n <= N; ++n)
                v[k][n] = s[n * kLanes];
        }
#pragma unroll
        for (int k = 0; k < kFoldGroup; ++k)
            fold_part_summary<N>(h, v[k], pow_path, A2, A2_0);
    }
    for (; k0 < count; ++k0) {
        const float *s = sbase + (int64_t)(first + k0 * dir) * (N + 1) * kLanes;
        float v[N + 1];
#pragma unroll
        for (int n = 0; n <= N; ++n)
            v[n] = s[n * kLanes];
        fold_part_summary<N>(h, v, pow_path, A2, A2_0);
    }
}

// Occupancy target: four waves per SIMD (at most 128 VGPRs) for N <= 16;
// three (at most 168 VGPRs) for the exact-ZOH variants, whose per-state
// coefficients would spill at 128.  (The conv variant spills a few registers
// at four waves and is still faster there than at three: measured.)  N = 32:
// two waves (256 VGPRs, a few spilled: batch 8, L 2048, D 1536 433 -> 274 us
// against one wave), one for exact ZOH; N = 64: one.
template <int N, int VAR>
constexpr int waves_per_eu()
{
    if (N > 32 || (N > 16 && (VAR & kVarZoh) != 0))
        return 1;
    if (N > 16)
        return 2;
    return (VAR & kVarZoh) != 0 ? 3 : 4;
}

// FIX = 0: the gate and the softplus switch are read at run time (the
// variants, the summary pass); FIX = 1 + 2 gated + softplus: both fixed at
// compile time (the main pass of the default forward and of reverse alone,
// whose host knows them): one recurrence loop per kernel instead of eight
// gives the register allocator less to share (main pass 70.8 -> 69.5 us on
// batch 8, L 2048, D 1536, measured).
template <int N, bool SUMMARY, int VAR, typename TIO, int FIX = 0>
__global__ __launch_bounds__(kLanes * kWavesPerBlock)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<N, VAR>()))) void fwd_stream_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    TIO *__restrict__ y, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ h0,
    float *__restrict__ h_last, float *__restrict__ summ, const float *__restrict__ entry,
    int64_t L, int64_t dim, int64_t groups, int parts, int64_t part_len, ExtParams ext)
{
    constexpr bool EXT = (VAR & kVarExt) != 0;
    constexpr bool ZOH = (VAR & kVarZoh) != 0;
    constexpr bool CONV = (VAR & kVarConv) != 0;
    const int lane = threadIdx.x & (kLanes - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves_parts = SUMMARY ? parts - 1 : parts;
    if (gw >= groups * waves_parts)
        return;   // whole wave: waves never synchronise with each other
    const int part = (int)(gw / groups);
    const int64_t grp = gw % groups;
    const int64_t groups_per_row = (dim + kLanes - 1) / kLanes;

    WaveCtx c;
    c.b = grp / groups_per_row;
    c.bL = c.b * L;
    c.d0 = (grp % groups_per_row) * kLanes;
    c.L = L;
    c.dim = dim;
    c.l_begin = (int64_t)part * part_len;
    c.l_end = c.l_begin + part_len < L ? c.l_begin + part_len : L;
    c.voff = lane * (int)sizeof(TIO);
    c.row_bytes = (int)(dim * (int64_t)sizeof(TIO));
    const bool active = c.d0 + lane < dim;
    const int64_t d = active ? c.d0 + lane : dim - 1;
    c.voff_store = active ? c.voff : kStoreOffsetOutOfRange;
    c.rev = (VAR & kVarRev) != 0 ? 1 : EXT ? ext.rev : 0;
    c.softplus = delta_softplus;

    const float A0 = A[d * N];
    bool structured = true;
    float A2[N], invA[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        invA[n] = ZOH ? 1.0f / an : 0.0f;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    const bool pow_path = __all(structured);
    c.A2_0 = A0 * kLog2e;
    c.invA0 = invA[0];
    c.bias = delta_bias ? delta_bias[d] : 0.0f;
    c.Dd = (!SUMMARY && D_skip) ? D_skip[d] : 0.0f;

    // Conv prologue: taps, and the raw inputs of the steps before the part.
    float win[kMaxConv - 1];
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j)
        win[j] = 0.0f;
    if constexpr (CONV) {
        conv_taps(c, ext, d);
        conv_window<VAR>(win, c, u, d);
    }

    // Entry state: zero for a summary; for the main pass h0 (or zero) carried
    // through the summaries of the parts before this one: folded by the carry
    // kernel (entry), or here when the sequence has only a few parts (no
    // carry launch; entry null).
    float h[N];
    if (!SUMMARY && entry) {
        load_entry<N>(h, entry, grp, parts, part, lane);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = (!SUMMARY && h0) ? h0[(c.b * dim + d) * N + n] : 0.0f;
        if (!SUMMARY)
            fold_summaries<N>(h, summ + (grp * (parts - 1)) * (N + 1) * kLanes + lane, 0, part, 1,
                              pow_path, A2, c.A2_0);
    }

    float sdelta = 0.0f;
    const bool gated = !SUMMARY && z != nullptr;
    float *ck = nullptr;
    if constexpr ((VAR & kVarKeep) != 0 && !SUMMARY)
        ck = ext.ckpt + grp * ext.nck * (N * kLanes) + lane;
#define SELSCAN_RUN(G, SP, PW)                                                                    \
    run_part<N, SUMMARY, G, SP, PW, VAR>(u, delta, z, y, Bm, Cm, c, A2, invA, h, sdelta, win, ck)
    if (SUMMARY && pow_path) {
        if (EXT || delta_softplus)
            summary_part_rev<N, true, VAR>(u, delta, Bm, c, win, h, sdelta);
        else
            summary_part_rev<N, false, VAR>(u, delta, Bm, c, win, h, sdelta);
    } else if (FIX != 0) {
        constexpr bool FG = ((FIX - 1) & 2) != 0, FS = ((FIX - 1) & 1) != 0;
        if (pow_path) SELSCAN_RUN(FG, FS, true); else SELSCAN_RUN(FG, FS, false);
    } else if (gated) {
        if (EXT || delta_softplus) {
            if (pow_path) SELSCAN_RUN(true, true, true); else SELSCAN_RUN(true, true, false);
        } else {
            if (pow_path) SELSCAN_RUN(true, false, true); else SELSCAN_RUN(true, false, false);
        }
    } else {
        if (EXT || delta_softplus) {
            if (pow_path) SELSCAN_RUN(false, true, true); else SELSCAN_RUN(false, true, false);
        } else {
            if (pow_path) SELSCAN_RUN(false, false, true); else SELSCAN_RUN(false, false, false);
        }
    }
#undef SELSCAN_RUN

    if (SUMMARY) {
        float *o = summ + ((grp * (parts - 1) + part) * (N + 1)) * kLanes + lane;
        o[0] = sdelta;
#pragma unroll
        for (int n = 0; n < N; ++n)
            o[(n + 1) * kLanes] = h[n];
    } else if (h_last && active && part == parts - 1) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h_last[(c.b * dim + d) * N + n] = h[n];
    }
}

inline float *summary_buffer(void *workspace)
{
    return (float *)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
}

// Entry states after the summaries: (groups, parts, N, 64) fp32.
inline float *entry_buffer(void *workspace, const StreamPlan &p, int64_t N)
{
    const size_t summ = (size_t)p.groups * (p.parts > 1 ? p.parts - 1 : 0) * (N + 1) * kLanes * 4;
    return (float *)((char *)summary_buffer(workspace) + ((summ + 255) & ~(size_t)255));
}

// The two-level carry's block buffers, after the entry states.
inline float *carry_scratch(void *workspace, const StreamPlan &p, int64_t N)
{
    const size_t entry = (size_t)p.groups * p.parts * N * kLanes * 4;
    return (float *)((char *)entry_buffer(workspace, p, N) + ((entry + 255) & ~(size_t)255));
}

// Summary pass (when the sequence is split), then the main pass, on one stream.
template <int N, int VAR, typename TIO>
hipError_t launch_n(const FwdArgs &a, const ExtParams &ext, const StreamPlan &p, float *summ,
                    float *entry, hipStream_t s)
{
    if (p.parts > 1) {
        const int64_t waves = p.groups * (p.parts - 1);
        hipLaunchKernelGGL((fwd_stream_kernel<N, true, VAR & ~kVarKeep, TIO>),
                           dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                           dim3(kLanes * kWavesPerBlock), 0, s, (const TIO *)a.u,
                           (const TIO *)a.delta, (const TIO *)nullptr, (TIO *)nullptr, a.A,
                           (const TIO *)a.Bm, (const TIO *)a.Cm, (const float *)nullptr,
                           a.delta_bias, a.delta_softplus, (const float *)nullptr,
                           (float *)nullptr, summ, (const float *)nullptr, a.L, a.dim, p.groups,
                           p.parts, p.part_len, ext);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (p.parts > kFoldInKernelMaxParts) {
            if (!entry)
                return hipErrorInvalidValue;   // the carry needs the entry buffer
            e = launch_fwd_carry(summ, a.h0, a.A, entry, a.batch, a.dim, N, p.parts, 0,
                                 carry_scratch(a.workspace, p, N), s);
            if (e != hipSuccess)
                return e;
        }
    }
    const int64_t waves = p.groups * p.parts;
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kLanes * kWavesPerBlock);
#define SELSCAN_MAIN(FX)                                                                          \
    hipLaunchKernelGGL((fwd_stream_kernel<N, false, VAR, TIO, FX>), grid, block, 0, s,              \
                       (const TIO *)a.u, (const TIO *)a.delta, (const TIO *)a.z, (TIO *)a.y, a.A,  \
                       (const TIO *)a.Bm, (const TIO *)a.Cm, a.D_skip, a.delta_bias,              \
                       a.delta_softplus, a.h0, a.h_last, summ,                                    \
                       (const float *)(p.parts > kFoldInKernelMaxParts ? entry : nullptr), a.L,   \
                       a.dim, p.groups, p.parts, p.part_len, ext)
    if constexpr ((VAR & ~kVarKeep) == 0 || (VAR & ~kVarKeep) == kVarRev) {
        const int fx = 1 + (a.z ? 2 : 0) + (a.delta_softplus ? 1 : 0);
        if (fx == 4) SELSCAN_MAIN(4); else if (fx == 3) SELSCAN_MAIN(3);
        else if (fx == 2) SELSCAN_MAIN(2); else SELSCAN_MAIN(1);
    } else {
        SELSCAN_MAIN(0);
    }
#undef SELSCAN_MAIN
    return hipGetLastError();
}

// Summary pass alone of a variant forward, for a given plan (the backward's).
template <int N, bool ZOH>
hipError_t launch_ext_summaries(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                float *summ, hipStream_t s)
{
    const int64_t waves = p.groups * (p.parts - 1);
    if (waves <= 0)
        return hipSuccess;
    ExtParams x{};
    x.conv_w = e.conv_k > 0 ? e.conv_w : nullptr;
    x.conv_b = e.conv_k > 0 ? e.conv_b : nullptr;
    x.conv_k = e.conv_k;
    x.rev = (e.flags & kFwdFlagReverse) ? 1 : 0;
    constexpr int V = kVarExt | (ZOH ? kVarZoh : 0);
    const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kLanes * kWavesPerBlock);
#define SELSCAN_SUMM(VV, T)                                                                       \
    hipLaunchKernelGGL((fwd_stream_kernel<N, true, VV, T>), grid, block, 0, s, (const T *)a.u,     \
                       (const T *)a.delta, (const T *)nullptr, (T *)nullptr, a.A,                 \
                       (const T *)a.Bm, (const T *)a.Cm, (const float *)nullptr, a.delta_bias,   \
                       a.delta_softplus, (const float *)nullptr, (float *)nullptr, summ,          \
                       (const float *)nullptr, a.L, a.dim, p.groups, p.parts, p.part_len, x)
    if (a.dtype == 1) {
        if (e.conv_k > 0) SELSCAN_SUMM(V | kVarConv, uint16_t); else SELSCAN_SUMM(V, uint16_t);
    } else {
        if (e.conv_k > 0) SELSCAN_SUMM(V | kVarConv, float); else SELSCAN_SUMM(V, float);
    }
#undef SELSCAN_SUMM
    return hipGetLastError();
}

// Variant forward for one N and one B_bar form (ZOH: exact zero-order hold):
// picks the instantiation from the conv width and the dtype.
// The variants in the forward direction, with the direction and the
// softplus switch fixed at compile time (conv, ZOH, ZOH + conv; the plain
// case is the default forward).  Instantiated explicitly in the
// fwd_stream_ext_n*_fixed.hip units, so that they compile in parallel with
// the reverse-direction ones.
template <int N, bool ZOH, typename TIO>
hipError_t launch_ext_fixed(const FwdArgs &a, const ExtParams &x, const StreamPlan &p,
                            float *summ, float *entry, hipStream_t s)
{
    constexpr int VF = ZOH ? kVarZoh : 0;
    if (x.conv_k > 0)
        return launch_n<N, VF | kVarConv, TIO>(a, x, p, summ, entry, s);
    if constexpr (ZOH)
        return launch_n<N, VF, TIO>(a, x, p, summ, entry, s);
    return hipErrorInvalidValue;   // no variant: selscan_fwd_ex runs the default forward
}

template <int N, bool ZOH>
hipError_t launch_ext(const FwdArgs &a, const FwdExt &e, hipStream_t s)
{
    constexpr int V0 = kVarExt | (ZOH ? kVarZoh : 0);
    float *summ = summary_buffer(a.workspace);
    const bool bf = a.dtype == 1;
    if constexpr (!ZOH) {
        if (e.conv_k == 0 && (e.flags & kFwdFlagReverse)) {
            // reverse alone: the default's plan, carry kernel and code with the
            // addressing mirrored (157 -> 134..142 us on batch 8, L 2048,
            // D 1536, N 16, against the run-time direction)
            const StreamPlan p = default_fwd_plan(a.batch, a.L, a.dim);
            float *entry = entry_buffer(a.workspace, p, N);
            ExtParams none{};
            return bf ? launch_n<N, kVarRev, uint16_t>(a, none, p, summ, entry, s)
                      : launch_n<N, kVarRev, float>(a, none, p, summ, entry, s);
        }
    }
    const int occupancy = e.conv_k > 0 ? waves_per_eu<N, V0 | kVarConv>() : waves_per_eu<N, V0>();
    const StreamPlan p = make_stream_plan(a.batch, a.L, a.dim, occupancy);
    float *entry = entry_buffer(a.workspace, p, N);
    ExtParams x{};
    x.conv_w = e.conv_k > 0 ? e.conv_w : nullptr;
    x.conv_b = e.conv_k > 0 ? e.conv_b : nullptr;
    x.conv_k = e.conv_k;
    x.rev = (e.flags & kFwdFlagReverse) ? 1 : 0;
    if (!x.rev)
        return bf ? launch_ext_fixed<N, ZOH, uint16_t>(a, x, p, summ, entry, s)
                  : launch_ext_fixed<N, ZOH, float>(a, x, p, summ, entry, s);
    // reverse with the conv prologue or exact ZOH: the direction fixed at
    // compile time as well (kVarRev; the softplus switch and the gate chosen
    // per launch, as in the forward-direction variants)
    constexpr int VR = kVarRev | (ZOH ? kVarZoh : 0);
    if (e.conv_k > 0)
        return bf ? launch_n<N, VR | kVarConv, uint16_t>(a, x, p, summ, entry, s)
                  : launch_n<N, VR | kVarConv, float>(a, x, p, summ, entry, s);
    return bf ? launch_n<N, VR, uint16_t>(a, x, p, summ, entry, s)
              : launch_n<N, VR, float>(a, x, p, summ, entry, s);
}

} // namespace stream
} // namespace selscan
