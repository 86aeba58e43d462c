// Streaming selective-scan forward for gfx950 (default forward path).
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
// a zero state and stores (sum of Delta over the part, end state); the main
// pass starts part p from h0 folded through the summaries of parts 0..p-1
// with the associative operator (a, b) o (c, d) = (a c, a d + b) of the
// selection-mechanism article (discosf.com) §3.1, where the decay of a whole
// part is exp(A sum Delta).
//
// Structured A: when every A[d, n] equals (n+1) A[d, 0] exactly (the S4D-real
// initialisation A = -exp(log(1..N)) of the tutorial's §4.2 listing),
// exp(Delta A[d, n]) = r^(n+1) with r = exp(Delta A[d, 0]), one multiply per
// (t, n) instead of a multiply and an exp2.  A wave uses it only if all its
// channels qualify; any other A takes the exp2 path.
#include "buffer_io.hpp"
#include "device_math.hpp"
#include "kernels.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace selscan {
namespace {

constexpr int kLanes = 64;
constexpr int kWavesPerBlock = 4;
constexpr int TT = 4;   // timesteps per prefetch buffer, main pass
constexpr int TTS = 8;  // timesteps per prefetch buffer, summary pass
// A store offset past the byte range of every output descriptor (a chunk's
// range is at most TT * dim * 4 bytes, and dim * 4 < 2^26 is checked on the
// host), so stores from lanes past dim are dropped by the hardware.
constexpr int kStoreOffsetOutOfRange = 1 << 30;

template <int TTc>
struct ChunkT {
    uint32_t u[TTc], x[TTc], z[TTc];   // raw element bits, widened at use
};
using Chunk = ChunkT<TT>;

struct WaveCtx {
    int64_t b, d0, L, dim, l_begin, l_end;
    int voff, row_bytes;
    int voff_store;    // voff, or an offset past every descriptor range for lanes past dim
    float bias, Dd, A2_0;
};

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

template <bool GATED, int TTc, typename TIO>
__device__ __forceinline__ void load_chunk(ChunkT<TTc> &ch, const TIO *u, const TIO *delta,
                                           const TIO *z, const WaveCtx &c, int64_t t0)
{
    constexpr int TT = TTc;
    int64_t rows = c.l_end - t0;
    rows = rows < 0 ? 0 : (rows > TT ? TT : rows);
    if (t0 < c.l_begin)
        rows = 0;
    const int64_t elem = (c.b * c.L + t0) * c.dim + c.d0;
    // A chunk outside the part has an empty range: its loads return 0 and
    // read nothing (the prefetch runs one chunk past either end).
    const int64_t bytes = rows > 0 ? (rows * c.dim - c.d0) * (int64_t)sizeof(TIO) : 0;
    const int64_t safe_elem = rows > 0 ? elem : 0;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(delta + safe_elem, bytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(u + safe_elem, bytes);
#pragma unroll
    for (int i = 0; i < TT; ++i)
        ch.x[i] = buf_load_raw(rd, c.voff, i * c.row_bytes, delta);
#pragma unroll
    for (int i = 0; i < TT; ++i)
        ch.u[i] = buf_load_raw(ru, c.voff, i * c.row_bytes, u);
    if (GATED) {
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + safe_elem, bytes);
#pragma unroll
        for (int i = 0; i < TT; ++i)
            ch.z[i] = buf_load_raw(rz, c.voff, i * c.row_bytes, z);
    }
}

// TT steps of the recurrence on one prefetched chunk.  FULL: all TT steps are
// inside the range (no per-step check); otherwise steps past the end are the
// identity element (Delta = 0).  The B_t / C_t rows of step i+1 are fetched
// (scalar loads) while step i computes.  The loop body has no branch, so the
// scheduler is free to move loads ahead.
template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, bool FULL, typename TIO>
__device__ __forceinline__ void run_chunk(const Chunk &ch, const TIO *Bm, const TIO *Cm, TIO *y,
                                          const WaveCtx &c, int64_t t0,
                                          const float (&A2)[N], float (&h)[N], float &sdelta)
{
    const int rows = FULL ? TT : (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    const int64_t elem = (c.b * c.L + t0) * c.dim + c.d0;
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(SUMMARY ? nullptr : y + elem, SUMMARY ? 0 : (rows * c.dim - c.d0) * (int64_t)sizeof(TIO));
    const int64_t row0 = c.b * c.L + t0;
    const int64_t row_last = c.b * c.L + c.L - 1;
    RowRaw<N, TIO> bcur, ccur, bnxt, cnxt;
    fetch_row(bcur, Bm, row0);
    if (!SUMMARY)
        fetch_row(ccur, Cm, row0);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        if (i + 1 < TT) {
            // rows past L are clamped (padding steps, never stored)
            const int64_t rn = (FULL || row0 + i + 1 <= row_last) ? row0 + i + 1 : row_last;
            fetch_row(bnxt, Bm, rn);
            if (!SUMMARY)
                fetch_row(cnxt, Cm, rn);
        }
        const bool valid = FULL || i < rows;
        const float ut = raw_to_f32(ch.u[i], tag<TIO>());
        const float x = raw_to_f32(ch.x[i], tag<TIO>()) + c.bias;
        float dt = SOFTPLUS ? softplus(x) : x;
        if (!FULL)
            dt = valid ? dt : 0.0f;        // padding steps are the identity (1, 0)
        const float du = dt * ut;
        float yv = c.Dd * ut;
        const float r = POW ? hw_exp2(dt * c.A2_0) : 0.0f;
        float pw = 1.0f;
        if (SUMMARY)
            sdelta += dt;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float a = POW ? (pw *= r) : hw_exp2(dt * A2[n]);
            h[n] = fmaf(a, h[n], du * row_val<N>(bcur, n));
            if (!SUMMARY)
                yv = fmaf(row_val<N>(ccur, n), h[n], yv);
        }
        if (!SUMMARY) {
            if (GATED)
                yv *= silu(raw_to_f32(ch.z[i], tag<TIO>()));
            // rows past the end and lanes past dim fall outside the descriptor
            buf_store(ry, c.voff_store, i * c.row_bytes, yv, y);
        }
        if (i + 1 < TT) {
            bcur = bnxt;
            if (!SUMMARY)
                ccur = cnxt;
        }
    }
}

template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, typename TIO>
__device__ __forceinline__ void run_any_chunk(const Chunk &ch, const TIO *Bm, const TIO *Cm, TIO *y,
                                              const WaveCtx &c, int64_t t0,
                                              const float (&A2)[N], float (&h)[N], float &sdelta)
{
    if (t0 + TT <= c.l_end)
        run_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, true>(ch, Bm, Cm, y, c, t0, A2, h, sdelta);
    else
        run_chunk<N, SUMMARY, GATED, SOFTPLUS, POW, false>(ch, Bm, Cm, y, c, t0, A2, h, sdelta);
}

// Forward walk over the part (main pass, and the summary for general A).
template <int N, bool SUMMARY, bool GATED, bool SOFTPLUS, bool POW, typename TIO>
__device__ __forceinline__ void run_part(const TIO *u, const TIO *delta, const TIO *z, TIO *y,
                                         const TIO *Bm, const TIO *Cm, const WaveCtx &c,
                                         const float (&A2)[N], float (&h)[N], float &sdelta)
{
    Chunk A, B;
    int64_t t0 = c.l_begin;
    load_chunk<GATED>(A, u, delta, z, c, t0);
    for (;;) {
        load_chunk<GATED>(B, u, delta, z, c, t0 + TT);
        run_any_chunk<N, SUMMARY, GATED, SOFTPLUS, POW>(A, Bm, Cm, y, c, t0, A2, h, sdelta);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
        load_chunk<GATED>(A, u, delta, z, c, t0 + TT);
        run_any_chunk<N, SUMMARY, GATED, SOFTPLUS, POW>(B, Bm, Cm, y, c, t0, A2, h, sdelta);
        t0 += TT;
        if (t0 >= c.l_end)
            break;
    }
}

// Summary of a part for structured A, walking the part backwards in time.
// The end state from zero is x[n] = sum_t Q_t^(n+1) Delta_t u_t B_t[n], with
// Q_t = prod_{s>t} r_s and r_s = exp(Delta_s A[d,0]).  Walking backwards, Q
// is one running product and Delta_t u_t Q_t^(n+1) one multiply per n, so a
// (t, n) costs a multiply and an FMA (the forward walk needs three ops).
template <int N, bool SOFTPLUS, bool FULL, typename TIO>
__device__ __forceinline__ void summary_chunk_rev(const ChunkT<TTS> &ch, const TIO *Bm,
                                                  const WaveCtx &c, int64_t t0, float &Q,
                                                  float (&x)[N], float &sdelta)
{
    constexpr int TT = TTS;
    const int rows = FULL ? TT : (int)(c.l_end - t0 < TT ? c.l_end - t0 : TT);
    const int64_t row0 = c.b * c.L + t0;
    // B_t row of step i-1 is fetched (scalar loads) while step i computes.
    RowRaw<N, TIO> bcur, bnxt;
    fetch_row(bcur, Bm, row0 + (FULL ? TT - 1 : rows - 1));
#pragma unroll
    for (int i = TT - 1; i >= 0; --i) {
        if (!FULL && i >= rows)
            continue;   // uniform: steps past the end contribute nothing
        if (i > 0)
            fetch_row(bnxt, Bm, row0 + i - 1);
        const float ut = raw_to_f32(ch.u[i], tag<TIO>());
        const float xr = raw_to_f32(ch.x[i], tag<TIO>()) + c.bias;
        const float dt = SOFTPLUS ? softplus(xr) : xr;
        sdelta += dt;
        float g = dt * ut * Q;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            if (n)
                g *= Q;
            x[n] = fmaf(g, row_val<N>(bcur, n), x[n]);
        }
        Q *= hw_exp2(dt * c.A2_0);
        if (i > 0)
            bcur = bnxt;
    }
}

template <int N, bool SOFTPLUS, typename TIO>
__device__ __forceinline__ void summary_part_rev(const TIO *u, const TIO *delta, const TIO *Bm,
                                                 const WaveCtx &c, float (&x)[N], float &sdelta)
{
    constexpr int TT = TTS;
    const int64_t nchunks = (c.l_end - c.l_begin + TT - 1) / TT;
    ChunkT<TTS> A, B;
    float Q = 1.0f;
    int64_t k = nchunks - 1;
    int64_t t0 = c.l_begin + k * TT;
    load_chunk<false>(A, u, delta, (const TIO *)nullptr, c, t0);
    // the last chunk may be partial; every other chunk is full
    load_chunk<false>(B, u, delta, (const TIO *)nullptr, c, t0 - TT);
    if (t0 + TT <= c.l_end)
        summary_chunk_rev<N, SOFTPLUS, true>(A, Bm, c, t0, Q, x, sdelta);
    else
        summary_chunk_rev<N, SOFTPLUS, false>(A, Bm, c, t0, Q, x, sdelta);
    for (;;) {
        if (--k < 0)
            break;
        t0 -= TT;
        load_chunk<false>(A, u, delta, (const TIO *)nullptr, c, t0 - TT);
        summary_chunk_rev<N, SOFTPLUS, true>(B, Bm, c, t0, Q, x, sdelta);
        if (--k < 0)
            break;
        t0 -= TT;
        load_chunk<false>(B, u, delta, (const TIO *)nullptr, c, t0 - TT);
        summary_chunk_rev<N, SOFTPLUS, true>(A, Bm, c, t0, Q, x, sdelta);
    }
}

// At most 128 VGPRs, so that four waves fit on each SIMD (N <= 16).
template <int N, bool SUMMARY, typename TIO>
__global__ __launch_bounds__(kLanes * kWavesPerBlock)
__attribute__((amdgpu_waves_per_eu(N <= 16 ? 4 : 1))) void fwd_stream_kernel(
    const TIO *__restrict__ u, const TIO *__restrict__ delta, const TIO *__restrict__ z,
    TIO *__restrict__ y, const float *__restrict__ A, const TIO *__restrict__ Bm,
    const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
    const float *__restrict__ delta_bias, int delta_softplus, const float *__restrict__ h0,
    float *__restrict__ h_last, float *__restrict__ summ, int64_t L, int64_t dim,
    int64_t groups, int parts, int64_t part_len)
{
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

    const float A0 = A[d * N];
    bool structured = true;
    float A2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    const bool pow_path = __all(structured);
    c.A2_0 = A0 * kLog2e;
    c.bias = delta_bias ? delta_bias[d] : 0.0f;
    c.Dd = (!SUMMARY && D_skip) ? D_skip[d] : 0.0f;

    // Entry state: zero for a summary; for the main pass h0 (or zero) carried
    // through the summaries of the parts before this one.
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n)
        h[n] = (!SUMMARY && h0) ? h0[(c.b * dim + d) * N + n] : 0.0f;
    if (!SUMMARY) {
        // h <- exp(A S) h + x for each earlier part (S = its sum of Delta, x =
        // its end state from zero); for structured A, exp(A[d,n] S) = e^(n+1).
        for (int q = 0; q < part; ++q) {
            const float *s = summ + ((grp * (parts - 1) + q) * (N + 1)) * kLanes + lane;
            const float S = s[0];
            if (pow_path) {
                const float e = hw_exp2(c.A2_0 * S);
                float pw = 1.0f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    pw *= e;
                    h[n] = fmaf(pw, h[n], s[(n + 1) * kLanes]);
                }
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n)
                    h[n] = fmaf(hw_exp2(A2[n] * S), h[n], s[(n + 1) * kLanes]);
            }
        }
    }

    float sdelta = 0.0f;
    const bool gated = !SUMMARY && z != nullptr;
#define SELSCAN_RUN(G, SP, PW)                                                                    \
    run_part<N, SUMMARY, G, SP, PW>(u, delta, z, y, Bm, Cm, c, A2, h, sdelta)
    if (SUMMARY && pow_path) {
        if (delta_softplus)
            summary_part_rev<N, true>(u, delta, Bm, c, h, sdelta);
        else
            summary_part_rev<N, false>(u, delta, Bm, c, h, sdelta);
    } else if (gated) {
        if (delta_softplus) {
            if (pow_path) SELSCAN_RUN(true, true, true); else SELSCAN_RUN(true, true, false);
        } else {
            if (pow_path) SELSCAN_RUN(true, false, true); else SELSCAN_RUN(true, false, false);
        }
    } else {
        if (delta_softplus) {
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

struct StreamPlan {
    int64_t groups, part_len;
    int parts;
};

// SELSCAN_STREAM_PARTS=P overrides the number of sequence parts (tuning knob).
// Default (measured on MI355X): about 4096 waves (4 per SIMD) when the channel
// groups are few; with many groups, at least 8 parts (when L allows), since
// smaller waves balance the tail of the grid better than fewer, longer ones.
StreamPlan make_stream_plan(int64_t batch, int64_t L, int64_t dim)
{
    StreamPlan p;
    p.groups = batch * ((dim + kLanes - 1) / kLanes);
    const int64_t target_waves = 4096;
    int64_t parts = (target_waves + p.groups - 1) / p.groups;
    const int64_t min_parts = L / 256 < 8 ? L / 256 : 8;
    if (parts < min_parts)
        parts = min_parts;
    const char *e = getenv("SELSCAN_STREAM_PARTS");
    long long ov = 0;
    if (e && sscanf(e, "%lld", &ov) == 1 && ov >= 1)
        parts = ov;
    const int64_t max_parts = (L + 4 * TT - 1) / (4 * TT);
    if (parts > max_parts)
        parts = max_parts;
    if (parts > 65536)
        parts = 65536;
    if (parts < 1)
        parts = 1;
    p.part_len = (L + parts - 1) / parts;
    p.part_len = (p.part_len + TT - 1) / TT * TT;
    p.parts = (int)((L + p.part_len - 1) / p.part_len);
    return p;
}

template <int N, typename TIO>
hipError_t launch_n(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    if (p.parts > 1) {
        const int64_t waves = p.groups * (p.parts - 1);
        hipLaunchKernelGGL((fwd_stream_kernel<N, true, TIO>),
                           dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                           dim3(kLanes * kWavesPerBlock), 0, s, (const TIO *)a.u,
                           (const TIO *)a.delta, (const TIO *)nullptr, (TIO *)nullptr, a.A,
                           (const TIO *)a.Bm, (const TIO *)a.Cm, (const float *)nullptr,
                           a.delta_bias, a.delta_softplus, (const float *)nullptr,
                           (float *)nullptr, summ, a.L, a.dim, p.groups, p.parts, p.part_len);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t waves = p.groups * p.parts;
    hipLaunchKernelGGL((fwd_stream_kernel<N, false, TIO>),
                       dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kLanes * kWavesPerBlock), 0, s, (const TIO *)a.u, (const TIO *)a.delta,
                       (const TIO *)a.z, (TIO *)a.y, a.A, (const TIO *)a.Bm, (const TIO *)a.Cm,
                       a.D_skip, a.delta_bias, a.delta_softplus, a.h0, a.h_last, summ, a.L,
                       a.dim, p.groups, p.parts, p.part_len);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_t(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    switch (a.N) {
    case 4: return launch_n<4, TIO>(a, p, summ, s);
    case 8: return launch_n<8, TIO>(a, p, summ, s);
    case 16: return launch_n<16, TIO>(a, p, summ, s);
    case 32: return launch_n<32, TIO>(a, p, summ, s);
    case 64: return launch_n<64, TIO>(a, p, summ, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

size_t fwd_stream_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    const StreamPlan p = make_stream_plan(batch, L, dim);
    return p.parts > 1 ? (size_t)p.groups * (p.parts - 1) * (N + 1) * kLanes * 4 + 256 : 0;
}

hipError_t launch_fwd_stream(const FwdArgs &a, hipStream_t stream)
{
    const StreamPlan p = make_stream_plan(a.batch, a.L, a.dim);
    float *summ = (float *)(((uintptr_t)a.workspace + 255) & ~(uintptr_t)255);
    return a.dtype == 1 ? launch_t<uint16_t>(a, p, summ, stream)
                        : launch_t<float>(a, p, summ, stream);
}

} // namespace selscan
