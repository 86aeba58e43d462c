// C-ABI layer of libselscan: host-side argument checks, launch planning and
// status codes.  The contract is documented in include/selscan.h.
//
// Every check below runs before the first HIP call, so an invalid call
// queues nothing and leaves outputs untouched (and works on a host without
// a GPU, which the CPU test suite relies on).
#include "../../include/selscan.h"
#include "kernels.hpp"

#include <mutex>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace {

thread_local int g_last_hip_error = 0;

bool supported_n(int64_t N)
{
    return N == 4 || N == 8 || N == 16 || N == 32 || N == 64;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest channel count: keeps every per-chunk buffer range and offset of the
// forward kernels within 32 bits (at most 16 timesteps x dim x 4 bytes < 2^30).
const int64_t kMaxDim = (int64_t)1 << 24;

// Every launch grid fits in 2^31 - 1 workgroups: the largest are one wave
// per (channel group, sequence part), parts <= ceil(L/16), and the carry
// kernel's N/4 workgroups per channel group.  (No shape whose arrays fit in
// device memory comes near this; the check keeps a larger one from being
// launched with a truncated grid.)
bool grids_fit(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    const int64_t groups = batch * ((dim + 63) / 64);
    const int64_t parts = (L + 15) / 16;
    const int64_t per_group = parts > N ? parts : N;
    return groups <= ((int64_t)1 << 31) / (per_group > 0 ? per_group : 1) - 1;
}

// Forward plans.  Default: the two-pass streaming kernel.  SELSCAN_FORCE_PLAN
// = lookback selects the single-pass streaming kernel with decoupled
// look-back; = chunked the workgroup-chunked kernel; = dpp the in-wave DPP
// scan over time (ablations; all compute the same recurrence).
enum Plan { PLAN_STREAM, PLAN_LOOKBACK, PLAN_CHUNKED, PLAN_DPP };

// Polls before a look-back wait gives up: SELSCAN_LOOKBACK_SPIN_LIMIT (a
// count >= 0), else the kernel's default (-1).
int lookback_spin_limit()
{
    const char *e = getenv("SELSCAN_LOOKBACK_SPIN_LIMIT");
    if (!e || !*e)
        return -1;
    char *end = nullptr;
    const long v = strtol(e, &end, 10);
    return (end && *end == 0 && v >= 0 && v <= 0x7fffffff) ? (int)v : -1;
}

Plan forced_plan()
{
    const char *e = getenv("SELSCAN_FORCE_PLAN");
    if (e && strcmp(e, "chunked") == 0)
        return PLAN_CHUNKED;
    if (e && strcmp(e, "lookback") == 0)
        return PLAN_LOOKBACK;
    if (e && strcmp(e, "dpp") == 0)
        return PLAN_DPP;
    return PLAN_STREAM;
}

// a * b * c without overflow past 2^62; returns -1 on overflow.
int64_t checked_count(int64_t a, int64_t b, int64_t c)
{
    const int64_t lim = (int64_t)1 << 62;
    if (a <= 0 || b <= 0 || c <= 0)
        return -1;
    if (a > lim / b)
        return -1;
    int64_t ab = a * b;
    if (ab > lim / c)
        return -1;
    return ab * c;
}

struct Range {
    const void *p;
    int64_t bytes;
};

bool overlaps(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0)
        return false;
    uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
    uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
    return a0 < b1 && b0 < a1;
}

int finish_launch(hipError_t e)
{
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SELSCAN_ERR_HIP;
    }
    return SELSCAN_OK;
}

} // namespace

namespace {

// The fixed device scratch of selscan_fwd_noalloc: its workspace, on every
// device the library runs on, for the life of the process.  Host code never
// uses the array's name as an address (on the host it is a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[SELSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there).  Returns the hipError_t of the lookup.
hipError_t scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Shared by selscan_fwd (ext == NULL), selscan_fwd_ex and (use_scratch)
// selscan_fwd_noalloc, whose workspace is the device's fixed scratch: there
// a shape needing more than SELSCAN_NOALLOC_SCRATCH_BYTES is refused, and
// the scratch is looked up only after every argument check has passed.
// need_at_least: a larger workspace the call needs (selscan_fwd_ex keeping
// the backward's checkpoints needs a backward's).
int fwd_common(const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
               const float *D_skip, const void *z, const float *delta_bias, int delta_softplus,
               const float *h0, void *y, float *h_last, int64_t batch, int64_t L, int64_t dim,
               int64_t N, int dtype, const selscan::FwdExt *ext, void *workspace,
               size_t workspace_bytes, void *stream, bool use_scratch = false,
               size_t need_at_least = 0)
{
    if (dtype != SELSCAN_F32 && dtype != SELSCAN_BF16)
        return SELSCAN_ERR_DTYPE;
    const int64_t elems = checked_count(batch, L, dim);
    const int64_t bcn = checked_count(batch, L, N > 0 ? N : 1);
    const int64_t states = checked_count(batch, dim, N > 0 ? N : 1);
    if (elems < 0 || bcn < 0 || states < 0 || N < 1)
        return SELSCAN_ERR_SHAPE;
    if (!u || !delta || !A || !Bm || !Cm || !y)
        return SELSCAN_ERR_NULL;
    if (!supported_n(N) || dim > kMaxDim || !grids_fit(batch, L, dim, N))
        return SELSCAN_ERR_UNSUPPORTED;
    const float *conv_w = ext && ext->conv_k > 0 ? ext->conv_w : nullptr;
    const float *conv_b = ext && ext->conv_k > 0 ? ext->conv_b : nullptr;
    const int64_t conv_k = ext ? ext->conv_k : 0;
    if (ext && ext->conv_k > 0 && !conv_w)
        return SELSCAN_ERR_NULL;
    const void *all[] = {u, delta, A, Bm, Cm, D_skip, z, delta_bias, h0, y, h_last, workspace,
                         conv_w, conv_b};
    for (const void *p : all)
        if (p && !aligned16(p))
            return SELSCAN_ERR_UNSUPPORTED;
    size_t need = selscan_fwd_workspace_bytes(batch, L, dim, N, dtype);
    need = need > need_at_least ? need : need_at_least;
    if (use_scratch) {
        if (need > (size_t)SELSCAN_NOALLOC_SCRATCH_BYTES)
            return SELSCAN_ERR_TOO_LARGE;
        workspace = nullptr;   // the scratch, looked up below: nothing of the caller's
        workspace_bytes = 0;
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return SELSCAN_ERR_WORKSPACE;
    }

    const int64_t es = dtype == SELSCAN_BF16 ? 2 : 4;
    const Range ins[] = {{u, elems * es},     {delta, elems * es},     {A, dim * N * 4},
                         {Bm, bcn * es},      {Cm, bcn * es},          {D_skip, dim * 4},
                         {z, elems * es},     {delta_bias, dim * 4},   {h0, states * 4},
                         {workspace, (int64_t)need}, {conv_w, dim * conv_k * 4},
                         {conv_b, dim * 4}};
    const Range outs[] = {{y, elems * es}, {h_last, states * 4}};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return SELSCAN_ERR_ALIAS;
    if (overlaps(outs[0], outs[1]))
        return SELSCAN_ERR_ALIAS;

    if (use_scratch) {
        // every argument check has passed: the first HIP call
        const hipError_t e = scratch_ptr(&workspace);
        if (e != hipSuccess)
            return finish_launch(e);
        workspace_bytes = SELSCAN_NOALLOC_SCRATCH_BYTES;
    }

    selscan::FwdArgs a;
    a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.D_skip = D_skip; a.z = z;
    a.delta_bias = delta_bias; a.delta_softplus = delta_softplus ? 1 : 0; a.h0 = h0; a.y = y;
    a.h_last = h_last; a.batch = batch; a.L = L; a.dim = dim; a.N = N; a.dtype = dtype;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    if (ext)
        return finish_launch(selscan::launch_fwd_stream_ext(a, *ext, (hipStream_t)stream));
    switch (forced_plan()) {
    case PLAN_CHUNKED:
        return finish_launch(selscan::launch_fwd_chunked(a, (hipStream_t)stream));
    case PLAN_DPP:
        return finish_launch(selscan::launch_fwd_dpp(a, (hipStream_t)stream));
    case PLAN_LOOKBACK:
        return finish_launch(
            selscan::launch_fwd_lookback(a, lookback_spin_limit(), (hipStream_t)stream));
    default:
        return finish_launch(selscan::launch_fwd_stream(a, (hipStream_t)stream));
    }
}

// Shared by selscan_bwd (ext == NULL) and selscan_bwd_ex.
int bwd_common(const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
               const float *D_skip, const void *z, const float *delta_bias, int delta_softplus,
               const float *h0, const void *dy, const float *dh_last, void *du, void *ddelta,
               float *dA, float *dB, float *dC, float *dD, void *dz, float *ddelta_bias,
               float *dh0, const selscan::FwdExt *ext, float *dconv_w, float *dconv_b,
               int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype, void *workspace,
               size_t workspace_bytes, void *stream)
{
    if (dtype != SELSCAN_F32 && dtype != SELSCAN_BF16)
        return SELSCAN_ERR_DTYPE;
    const int64_t elems = checked_count(batch, L, dim);
    const int64_t bcn = checked_count(batch, L, N > 0 ? N : 1);
    const int64_t states = checked_count(batch, dim, N > 0 ? N : 1);
    if (elems < 0 || bcn < 0 || states < 0 || N < 1)
        return SELSCAN_ERR_SHAPE;
    if (!u || !delta || !A || !Bm || !Cm || !dy || !du || !ddelta || !dA || !dB || !dC ||
        (z && !dz))
        return SELSCAN_ERR_NULL;
    if (!supported_n(N) || dim > kMaxDim || !grids_fit(batch, L, dim, N))
        return SELSCAN_ERR_UNSUPPORTED;
    if (!z)
        dz = nullptr;
    const int64_t conv_k = ext ? ext->conv_k : 0;
    const float *conv_w = conv_k > 0 ? ext->conv_w : nullptr;
    const float *conv_b = conv_k > 0 ? ext->conv_b : nullptr;
    if (conv_k > 0 && (!conv_w || !dconv_w))
        return SELSCAN_ERR_NULL;
    if (conv_k == 0)
        dconv_w = dconv_b = nullptr;
    const void *all[] = {u,  delta, A,  Bm, Cm, D_skip, z,  delta_bias,  h0,  dy,       dh_last,
                         du, ddelta, dA, dB, dC, dD,     dz, ddelta_bias, dh0, workspace,
                         conv_w, conv_b, dconv_w, dconv_b};
    for (const void *p : all)
        if (p && !aligned16(p))
            return SELSCAN_ERR_UNSUPPORTED;
    const size_t need = selscan_bwd_workspace_bytes(batch, L, dim, N, dtype);
    if (!workspace || workspace_bytes < need)
        return SELSCAN_ERR_WORKSPACE;

    const int64_t es = dtype == SELSCAN_BF16 ? 2 : 4;
    const Range ins[] = {{u, elems * es},       {delta, elems * es},   {A, dim * N * 4},
                         {Bm, bcn * es},        {Cm, bcn * es},        {D_skip, dim * 4},
                         {z, elems * es},       {delta_bias, dim * 4}, {h0, states * 4},
                         {dy, elems * es},      {dh_last, states * 4}, {workspace, (int64_t)need},
                         {conv_w, dim * conv_k * 4}, {conv_b, dim * 4}};
    const Range outs[] = {{du, elems * es}, {ddelta, elems * es}, {dA, dim * N * 4},
                          {dB, bcn * 4},    {dC, bcn * 4},        {dD, dim * 4},
                          {dz, elems * es}, {ddelta_bias, dim * 4}, {dh0, states * 4},
                          {dconv_w, dim * conv_k * 4}, {dconv_b, dim * 4}};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i))
                return SELSCAN_ERR_ALIAS;
    const int n_out = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < n_out; ++i)
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j]))
                return SELSCAN_ERR_ALIAS;

    selscan::BwdArgs a;
    selscan::FwdArgs &f = a.fwd;
    f.u = u; f.delta = delta; f.A = A; f.Bm = Bm; f.Cm = Cm; f.D_skip = D_skip; f.z = z;
    f.delta_bias = delta_bias; f.delta_softplus = delta_softplus ? 1 : 0; f.h0 = h0;
    f.y = nullptr; f.h_last = nullptr; f.batch = batch; f.L = L; f.dim = dim; f.N = N;
    f.dtype = dtype; f.workspace = workspace; f.workspace_bytes = workspace_bytes;
    a.dy = dy; a.dh_last = dh_last; a.du = du; a.ddelta = ddelta; a.dz = dz; a.dA = dA;
    a.dB = dB; a.dC = dC; a.dD = dD; a.ddelta_bias = ddelta_bias; a.dh0 = dh0;
    a.dconv_w = dconv_w; a.dconv_b = dconv_b;
    return finish_launch(selscan::launch_bwd(a, ext, (hipStream_t)stream));
}

} // namespace

extern "C" {

int selscan_abi_version(void) { return SELSCAN_ABI_VERSION; }

const char *selscan_status_string(int status)
{
    switch (status) {
    case SELSCAN_OK: return "ok";
    case SELSCAN_ERR_NULL: return "a required pointer is NULL";
    case SELSCAN_ERR_SHAPE: return "a size is < 1 or an element count overflows";
    case SELSCAN_ERR_DTYPE: return "dtype is not SELSCAN_F32 or SELSCAN_BF16";
    case SELSCAN_ERR_UNSUPPORTED: return "unsupported N or a pointer not 16-byte aligned";
    case SELSCAN_ERR_WORKSPACE: return "workspace missing or too small";
    case SELSCAN_ERR_ALIAS: return "an output overlaps an input";
    case SELSCAN_ERR_HIP: return "a HIP runtime call failed";
    case SELSCAN_ERR_TIMEOUT: return "a bounded wait inside a kernel gave up; outputs are invalid";
    case SELSCAN_ERR_TOO_LARGE:
        return "the shape needs more workspace than the fixed scratch of selscan_fwd_noalloc";
    default: return "unknown status";
    }
}

int selscan_last_hip_error(void) { return g_last_hip_error; }

int selscan_fwd_status(const void *workspace, void *stream)
{
    if (forced_plan() != PLAN_LOOKBACK)
        return SELSCAN_OK;   // no other plan has a wait that can give up
    if (!workspace)
        return SELSCAN_ERR_NULL;
    const unsigned *base = (const unsigned *)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    unsigned word = 0;
    hipError_t e = hipMemcpyAsync(&word, base + selscan::kLookbackStatusWord, sizeof(word),
                                  hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return SELSCAN_ERR_HIP;
    }
    return word ? SELSCAN_ERR_TIMEOUT : SELSCAN_OK;
}

int selscan_supports_n(int64_t N) { return supported_n(N) ? 1 : 0; }

size_t selscan_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype)
{
    if ((dtype != SELSCAN_F32 && dtype != SELSCAN_BF16) || !supported_n(N) ||
        checked_count(batch, L, dim) < 0 || checked_count(batch, L, N) < 0 ||
        !grids_fit(batch, L, dim, N))
        return 0;
    const size_t a = selscan::fwd_chunked_workspace_bytes(batch, L, dim, N);
    const size_t b = selscan::fwd_stream_workspace_bytes(batch, L, dim, N);
    const size_t c = selscan::fwd_lookback_workspace_bytes(batch, L, dim, N);
    const size_t d = selscan::fwd_dpp_workspace_bytes(batch, L, dim, N);
    const size_t ab = a > b ? a : b;
    const size_t cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

int selscan_fwd(const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
                const float *D_skip, const void *z, const float *delta_bias, int delta_softplus,
                const float *h0, void *y, float *h_last, int64_t batch, int64_t L, int64_t dim,
                int64_t N, int dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return fwd_common(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, y, h_last,
                      batch, L, dim, N, dtype, nullptr, workspace, workspace_bytes, stream);
}

int selscan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *Bm,
                        const void *Cm, const float *D_skip, const void *z,
                        const float *delta_bias, int delta_softplus, const float *h0, void *y,
                        float *h_last, int64_t batch, int64_t L, int64_t dim, int64_t N,
                        int dtype, void *stream)
{
    return fwd_common(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, y, h_last,
                      batch, L, dim, N, dtype, nullptr, nullptr, 0, stream, true);
}

int selscan_fwd_ex(const void *u, const void *delta, const float *A, const void *Bm,
                   const void *Cm, const float *D_skip, const void *z, const float *delta_bias,
                   int delta_softplus, const float *h0, void *y, float *h_last, int64_t batch,
                   int64_t L, int64_t dim, int64_t N, int dtype, int flags,
                   const float *conv_weight, const float *conv_bias, int64_t conv_width,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (flags & ~(SELSCAN_FLAG_ZOH_EXACT | SELSCAN_FLAG_REVERSE | SELSCAN_FLAG_KEEP_CHECKPOINTS))
        return SELSCAN_ERR_UNSUPPORTED;
    if (conv_width < 0)
        return SELSCAN_ERR_SHAPE;
    if (conv_width > SELSCAN_MAX_CONV_WIDTH)
        return SELSCAN_ERR_UNSUPPORTED;
    // the checkpoints are kept by the plain forward or reverse alone
    const bool keep = (flags & SELSCAN_FLAG_KEEP_CHECKPOINTS) != 0;
    if (keep && ((flags & SELSCAN_FLAG_ZOH_EXACT) || conv_width > 0))
        return SELSCAN_ERR_UNSUPPORTED;
    selscan::FwdExt e;
    e.flags = (flags & SELSCAN_FLAG_ZOH_EXACT ? selscan::kFwdFlagZohExact : 0) |
              (flags & SELSCAN_FLAG_REVERSE ? selscan::kFwdFlagReverse : 0) |
              (keep ? selscan::kFwdFlagKeepCheckpoints : 0);
    e.conv_w = conv_weight;
    e.conv_b = conv_bias;
    e.conv_k = (int)conv_width;
    // with the checkpoints kept, the workspace is a backward's (a shape the
    // backward refuses has no such size: the argument checks then name the
    // error, or the workspace check fails, before any launch)
    const size_t need = keep ? selscan_bwd_workspace_bytes(batch, L, dim, N, dtype) : 0;
    return fwd_common(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, y, h_last,
                      batch, L, dim, N, dtype, &e, workspace, workspace_bytes, stream, false,
                      keep && need == 0 ? (size_t)-1 : need);
}

size_t selscan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype)
{
    if ((dtype != SELSCAN_F32 && dtype != SELSCAN_BF16) || !supported_n(N) ||
        checked_count(batch, L, dim) < 0 || checked_count(batch, L, N) < 0 || dim > kMaxDim ||
        !grids_fit(batch, L, dim, N))
        return 0;
    return selscan::bwd_workspace_bytes(batch, L, dim, N);
}

int selscan_bwd(const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
                const float *D_skip, const void *z, const float *delta_bias, int delta_softplus,
                const float *h0, const void *dy, const float *dh_last, void *du, void *ddelta,
                float *dA, float *dB, float *dC, float *dD, void *dz, float *ddelta_bias,
                float *dh0, int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_common(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, dy, dh_last,
                      du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nullptr, nullptr,
                      nullptr, batch, L, dim, N, dtype, workspace, workspace_bytes, stream);
}

int selscan_bwd_ex(const void *u, const void *delta, const float *A, const void *Bm,
                   const void *Cm, const float *D_skip, const void *z, const float *delta_bias,
                   int delta_softplus, const float *h0, const void *dy, const float *dh_last,
                   void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz,
                   float *ddelta_bias, float *dh0, int flags, const float *conv_weight,
                   const float *conv_bias, int64_t conv_width, float *dconv_weight,
                   float *dconv_bias, int64_t batch, int64_t L, int64_t dim, int64_t N, int dtype,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (flags & ~(SELSCAN_FLAG_ZOH_EXACT | SELSCAN_FLAG_REVERSE | SELSCAN_FLAG_REUSE_FWD_STATE |
                  SELSCAN_FLAG_KEEP_CHECKPOINTS))
        return SELSCAN_ERR_UNSUPPORTED;
    // kept checkpoints are read with the forward's part state (plain or
    // reverse alone: the ZOH and conv cases are refused with the reuse below)
    if ((flags & SELSCAN_FLAG_KEEP_CHECKPOINTS) && !(flags & SELSCAN_FLAG_REUSE_FWD_STATE))
        return SELSCAN_ERR_UNSUPPORTED;
    if (conv_width < 0)
        return SELSCAN_ERR_SHAPE;
    if (conv_width > SELSCAN_MAX_CONV_WIDTH)
        return SELSCAN_ERR_UNSUPPORTED;
    // the forward's part state has the backward's layout only where both run
    // the default plan: the plain forward and the reverse-alone variant
    if ((flags & SELSCAN_FLAG_REUSE_FWD_STATE) &&
        ((flags & SELSCAN_FLAG_ZOH_EXACT) || conv_width > 0))
        return SELSCAN_ERR_UNSUPPORTED;
    // a forced forward plan leaves another workspace layout (or none)
    if ((flags & SELSCAN_FLAG_REUSE_FWD_STATE) && forced_plan() != PLAN_STREAM)
        return SELSCAN_ERR_UNSUPPORTED;
    selscan::FwdExt e;
    e.flags = (flags & SELSCAN_FLAG_ZOH_EXACT ? selscan::kFwdFlagZohExact : 0) |
              (flags & SELSCAN_FLAG_REVERSE ? selscan::kFwdFlagReverse : 0) |
              (flags & SELSCAN_FLAG_REUSE_FWD_STATE ? selscan::kBwdFlagReuseFwdState : 0) |
              (flags & SELSCAN_FLAG_KEEP_CHECKPOINTS ? selscan::kFwdFlagKeepCheckpoints : 0);
    e.conv_w = conv_weight;
    e.conv_b = conv_bias;
    e.conv_k = (int)conv_width;
    return bwd_common(u, delta, A, Bm, Cm, D_skip, z, delta_bias, delta_softplus, h0, dy, dh_last,
                      du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, &e, dconv_weight,
                      dconv_bias, batch, L, dim, N, dtype, workspace, workspace_bytes, stream);
}

int selscan_state_update(float *state, const void *u, const void *delta, const float *A,
                         const void *Bm, const void *Cm, const float *D_skip, const void *z,
                         const float *delta_bias, int delta_softplus, void *y, int64_t batch,
                         int64_t dim, int64_t N, int dtype, void *stream)
{
    if (dtype != SELSCAN_F32 && dtype != SELSCAN_BF16)
        return SELSCAN_ERR_DTYPE;
    const int64_t elems = checked_count(batch, dim, 1);
    const int64_t states = checked_count(batch, dim, N > 0 ? N : 1);
    const int64_t bcn = checked_count(batch, N > 0 ? N : 1, 1);
    if (elems < 0 || states < 0 || bcn < 0 || N < 1)
        return SELSCAN_ERR_SHAPE;
    if (!state || !u || !delta || !A || !Bm || !Cm || !y)
        return SELSCAN_ERR_NULL;
    // 32-bit state indices in the kernel: batch * dim * N < 2^31
    if (!supported_n(N) || states >= ((int64_t)1 << 31))
        return SELSCAN_ERR_UNSUPPORTED;
    const void *all[] = {state, u, delta, A, Bm, Cm, D_skip, z, delta_bias, y};
    for (const void *p : all)
        if (p && !aligned16(p))
            return SELSCAN_ERR_UNSUPPORTED;

    const int64_t es = dtype == SELSCAN_BF16 ? 2 : 4;
    const Range ins[] = {{u, elems * es},  {delta, elems * es}, {A, dim * N * 4},
                         {Bm, bcn * es},   {Cm, bcn * es},      {D_skip, dim * 4},
                         {z, elems * es},  {delta_bias, dim * 4}};
    const Range st = {state, states * 4};
    const Range yo = {y, elems * es};
    for (const Range &i : ins)
        if (overlaps(st, i) || overlaps(yo, i))
            return SELSCAN_ERR_ALIAS;
    if (overlaps(st, yo))
        return SELSCAN_ERR_ALIAS;

    selscan::StepArgs a;
    a.state = state; a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm;
    a.D_skip = D_skip; a.z = z; a.delta_bias = delta_bias;
    a.delta_softplus = delta_softplus ? 1 : 0; a.y = y; a.batch = batch; a.dim = dim; a.N = N;
    a.dtype = dtype;
    return finish_launch(selscan::launch_state_update(a, (hipStream_t)stream));
}

} // extern "C"
