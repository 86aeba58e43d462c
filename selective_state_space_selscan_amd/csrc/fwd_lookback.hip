// Single-pass streaming forward with decoupled look-back (SELSCAN_FORCE_PLAN=lookback).
//
// The same per-wave work as the two-pass streaming forward (fwd_stream.hip),
// in one launch: every wave summarises its sequence part (sum of Delta and the
// end state from zero, the associative element of the part under the operator
// (a, b) o (c, d) = (a c, a d + b) of the selection-mechanism article
// (discosf.com) §3.1), publishes it, obtains its entry state by looking back
// over the parts before it, publishes its inclusive state (the true state at
// the end of its part), and then runs the part.  This is the chunked scan with
// a carry between blocks of the paper walkthrough (m.lqnn.cn) §3.2, with the
// carry passed through device memory instead of a grid-wide barrier.
//
// Look-back: wave p reads the flag of part p-1.  An inclusive state ends the
// walk; an aggregate is folded into the running composition of the parts
// between and the walk moves one part further back.  Parts are handed out in
// the order the waves start (a ticket counter), so a wave only waits for
// waves that started before it and never wait for it: every wait ends.  The
// waits are still bounded (a poll limit, kSpinLimit by default).  A wave
// whose wait gives up sets the status word of the workspace (read back by
// selscan_fwd_status) and poisons its state with NaN, so that its part and
// every later part of its group come out NaN rather than silently wrong.
//
// Memory ordering: a part's data is written with device-coherent (agent-scope)
// atomic stores; once they have completed (s_waitcnt) the part's flag is set
// with an atomic store.  A reader polls the flags with atomic loads until it
// meets an inclusive state (every flag it passed is at least an aggregate),
// then reads the data with device-coherent atomic loads, issued after the
// polls.  Agent-scope fences would instead write back and invalidate the
// per-XCD L2 caches on every publish and every read, which measured several
// times slower.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace {

using namespace stream;

constexpr unsigned kFlagAggregate = 1;
constexpr unsigned kFlagInclusive = 2;
constexpr int kSpinLimit = 1 << 20;

struct LookbackWs {
    unsigned *ticket;   // one counter, zero at launch
    unsigned *status;   // zero at launch; bit 0 set by a wave whose wait gave up
    unsigned *flags;    // (groups, parts), zero at launch
    float *agg;         // (groups, parts, N + 1, 64): sum of Delta, end state from zero
    float *incl;        // (groups, parts, N, 64): state at the end of the part
};

__global__ __launch_bounds__(256) void lookback_clear_kernel(unsigned *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

// Polls a flag (relaxed) until it is nonzero or `limit` polls pass (then 0).
__device__ __forceinline__ unsigned poll_flag(unsigned *f, int limit)
{
    unsigned v = 0;
    for (int it = 0; it < limit; ++it) {
        v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v != 0)
            break;
        __builtin_amdgcn_s_sleep(2);
    }
    return v;
}

// Cross-wave data goes through agent-scope (device-coherent) atomic loads and
// stores, so no fence has to write back or invalidate the per-XCD L2 caches.
__device__ __forceinline__ void put(float *p, float v)
{
    __hip_atomic_store(reinterpret_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get(const float *p)
{
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned *>(p),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Sets a part's flag once every lane's device-coherent stores have completed.
__device__ __forceinline__ void publish(unsigned *f, unsigned v)
{
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if ((threadIdx.x & (kLanes - 1)) == 0)
        __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// E[n] = exp(A[d,n] S): the decay over parts whose Delta sums to S.
template <int N>
__device__ __forceinline__ void decay(float (&E)[N], float S, bool pow_path,
                                      const float (&A2)[N], float A2_0)
{
    if (pow_path) {
        const float e = hw_exp2(A2_0 * S);
        float pw = 1.0f;
#pragma unroll
        for (int n = 0; n < N; ++n)
            E[n] = (pw *= e);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n)
            E[n] = hw_exp2(A2[n] * S);
    }
}

template <int N, typename TIO>
__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(N <= 16 ? 4 : 1)))
void fwd_lookback_kernel(const TIO *__restrict__ u, const TIO *__restrict__ delta,
                         const TIO *__restrict__ z, TIO *__restrict__ y,
                         const float *__restrict__ A, const TIO *__restrict__ Bm,
                         const TIO *__restrict__ Cm, const float *__restrict__ D_skip,
                         const float *__restrict__ delta_bias, int delta_softplus,
                         const float *__restrict__ h0, float *__restrict__ h_last, LookbackWs ws,
                         int64_t L, int64_t dim, int64_t groups, int parts, int64_t part_len,
                         int spin_limit)
{
    __shared__ unsigned s_ticket;
    if (threadIdx.x == 0)
        s_ticket = atomicAdd(ws.ticket, 1u);
    __syncthreads();
    const int64_t gw = s_ticket;
    if (gw >= groups * parts)
        return;
    const int lane = threadIdx.x & (kLanes - 1);
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
    c.rev = 0;
    c.softplus = delta_softplus;
    c.invA0 = 0.0f;
    c.cb = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j)
        c.cw[j] = 0.0f;

    const float A0 = A[d * N];
    bool structured = true;
    float A2[N], invA[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float an = A[d * N + n];
        A2[n] = an * kLog2e;
        invA[n] = 0.0f;
        structured = structured && (an == (float)(n + 1) * A0);
    }
    const bool pow_path = __all(structured);
    c.A2_0 = A0 * kLog2e;
    c.bias = delta_bias ? delta_bias[d] : 0.0f;
    float win[kMaxConv - 1] = {};

    const int64_t slot = grp * parts + part;
    float *agg = ws.agg + slot * (N + 1) * kLanes + lane;
    float *incl = ws.incl + slot * N * kLanes + lane;
    const bool last = part == parts - 1;

    // 1. this part's aggregate (not needed by anyone for the last part)
    float x[N], S = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n)
        x[n] = 0.0f;
    if (!last) {
        c.Dd = 0.0f;
        if (pow_path) {
            if (delta_softplus)
                summary_part_rev<N, true, 0>(u, delta, Bm, c, win, x, S);
            else
                summary_part_rev<N, false, 0>(u, delta, Bm, c, win, x, S);
        } else {
            if (delta_softplus)
                run_part<N, true, false, true, false, 0>(u, delta, z, y, Bm, Cm, c, A2, invA, x,
                                                         S, win);
            else
                run_part<N, true, false, false, false, 0>(u, delta, z, y, Bm, Cm, c, A2, invA,
                                                          x, S, win);
        }
        put(agg, S);
#pragma unroll
        for (int n = 0; n < N; ++n)
            put(agg + (n + 1) * kLanes, x[n]);
        publish(&ws.flags[slot], kFlagAggregate);
    }

    // 2. look back: compose the aggregates of parts q+1 .. part-1 (xa, Sa)
    //    until part q has its inclusive state (or q < 0: the entry is h0)
    float xa[N], Sa = 0.0f, hin[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        xa[n] = 0.0f;
        hin[n] = h0 ? h0[(c.b * dim + d) * N + n] : 0.0f;
    }
    // Find how far back to look with relaxed polls, then acquire once and
    // read the states: an acquire costs an L2 invalidation on this chip.
    int q_stop = -1;   // the part whose inclusive state ends the walk (-1: h0)
    bool gave_up = false;
    for (int q = part - 1; q >= 0; --q) {
        const unsigned f = poll_flag(&ws.flags[grp * parts + q], spin_limit);
        if (f == 0) {
            gave_up = true;   // part q never published within the limit
            break;
        }
        if (f == kFlagInclusive) {
            q_stop = q;
            break;
        }
    }
    if (gave_up) {
        if (lane == 0)
            __hip_atomic_fetch_or(ws.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        q_stop = part - 1;   // read nothing unpublished below: the state is poisoned instead
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // keeps the data reads below
    if (q_stop >= 0) {
        const float *qi = ws.incl + (grp * parts + q_stop) * N * kLanes + lane;
#pragma unroll
        for (int n = 0; n < N; ++n)
            hin[n] = get(qi + n * kLanes);
    }
    for (int q = part - 1; q > q_stop; --q) {
        // prepend part q: (Sq, xq) then (Sa, xa) = (Sq + Sa, exp(A Sa) xq + xa)
        const float *qa = ws.agg + (grp * parts + q) * (N + 1) * kLanes + lane;
        float E[N];
        decay<N>(E, Sa, pow_path, A2, c.A2_0);
#pragma unroll
        for (int n = 0; n < N; ++n)
            xa[n] = fmaf(E[n], get(qa + (n + 1) * kLanes), xa[n]);
        Sa += get(qa);
    }
    float h[N];
    {
        float E[N];
        decay<N>(E, Sa, pow_path, A2, c.A2_0);
        const float poison = gave_up ? __builtin_nanf("") : 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = fmaf(E[n], hin[n], xa[n]) + poison;
    }

    // 3. this part's inclusive state, for the parts after it
    if (!last) {
        float E[N];
        decay<N>(E, S, pow_path, A2, c.A2_0);
#pragma unroll
        for (int n = 0; n < N; ++n)
            put(incl + n * kLanes, fmaf(E[n], h[n], x[n]));
        publish(&ws.flags[slot], kFlagInclusive);
    }

    // 4. the part itself
    c.Dd = D_skip ? D_skip[d] : 0.0f;
    float sdelta = 0.0f;
    const bool gated = z != nullptr;
#define SELSCAN_RUN(G, SP, PW)                                                                    \
    run_part<N, false, G, SP, PW, 0>(u, delta, z, y, Bm, Cm, c, A2, invA, h, sdelta, win)
    if (gated) {
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
    if (h_last && active && last) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h_last[(c.b * dim + d) * N + n] = h[n];
    }
}

// The ticket counter and the status word lead the workspace (words 0 and 1
// of the aligned base: selscan_fwd_status reads word 1), then the flags.
struct LookbackLayout {
    size_t flags, agg, incl, total;   // byte offsets from the aligned base
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LookbackLayout lookback_layout(const StreamPlan &p, int64_t N)
{
    LookbackLayout w;
    const size_t slots = (size_t)p.groups * p.parts;
    w.flags = 0;
    w.agg = align256((kLookbackFlagsOffset + slots) * sizeof(unsigned));
    w.incl = align256(w.agg + slots * (N + 1) * kLanes * 4);
    w.total = align256(w.incl + slots * N * kLanes * 4) + 256;
    return w;
}

template <int N, typename TIO>
hipError_t launch_n(const FwdArgs &a, const StreamPlan &p, char *base, int spin_limit,
                    hipStream_t s)
{
    const LookbackLayout l = lookback_layout(p, N);
    LookbackWs ws;
    ws.ticket = (unsigned *)(base + l.flags);
    ws.status = ws.ticket + kLookbackStatusWord;
    ws.flags = ws.ticket + kLookbackFlagsOffset;
    ws.agg = (float *)(base + l.agg);
    ws.incl = (float *)(base + l.incl);
    const int64_t nflags = kLookbackFlagsOffset + p.groups * p.parts;
    hipLaunchKernelGGL(lookback_clear_kernel, dim3((unsigned)((nflags + 255) / 256)), dim3(256),
                       0, s, ws.ticket, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t waves = p.groups * p.parts;
    hipLaunchKernelGGL((fwd_lookback_kernel<N, TIO>), dim3((unsigned)waves), dim3(kLanes), 0, s,
                       (const TIO *)a.u, (const TIO *)a.delta, (const TIO *)a.z, (TIO *)a.y, a.A,
                       (const TIO *)a.Bm, (const TIO *)a.Cm, a.D_skip, a.delta_bias,
                       a.delta_softplus, a.h0, a.h_last, ws, a.L, a.dim, p.groups, p.parts,
                       p.part_len, spin_limit);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_t(const FwdArgs &a, const StreamPlan &p, char *base, int spin, hipStream_t s)
{
    switch (a.N) {
    case 4: return launch_n<4, TIO>(a, p, base, spin, s);
    case 8: return launch_n<8, TIO>(a, p, base, spin, s);
    case 16: return launch_n<16, TIO>(a, p, base, spin, s);
    case 32: return launch_n<32, TIO>(a, p, base, spin, s);
    case 64: return launch_n<64, TIO>(a, p, base, spin, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

size_t fwd_lookback_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    return lookback_layout(make_stream_plan(batch, L, dim), N).total;
}

hipError_t launch_fwd_lookback(const FwdArgs &a, int spin_limit, hipStream_t stream)
{
    const StreamPlan p = make_stream_plan(a.batch, a.L, a.dim);
    char *base = (char *)(((uintptr_t)a.workspace + 255) & ~(uintptr_t)255);
    const int spin = spin_limit >= 0 ? spin_limit : kSpinLimit;
    return a.dtype == 1 ? launch_t<uint16_t>(a, p, base, spin, stream)
                        : launch_t<float>(a, p, base, spin, stream);
}

} // namespace selscan
