// Streaming selective-scan forward: launch plan, the default instantiation
// (Euler B_bar = Delta B, forward direction, no prologue) and the dispatch of
// the variants.  The kernel itself is in fwd_stream_impl.hpp.
#include "fwd_stream_impl.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace selscan {

// SELSCAN_STREAM_PARTS=P overrides the number of sequence parts (tuning knob).
// Default (measured on MI355X): about one wave per wave slot of the chip (1024
// SIMDs x the kernel's waves per SIMD) when the channel groups are few; with
// many groups, at least 8 parts (when L allows), since smaller waves balance
// the tail of the grid better than fewer, longer ones.  Parts are whole
// multiples of kStreamTT steps and at least 4 of them long.
StreamPlan make_stream_plan(int64_t batch, int64_t L, int64_t dim, int waves_per_simd)
{
    constexpr int kLanes = stream::kLanes;
    constexpr int TT = kStreamTT;
    StreamPlan p;
    p.groups = batch * ((dim + kLanes - 1) / kLanes);
    const int64_t target_waves = 1024 * (int64_t)waves_per_simd;
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

size_t fwd_stream_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    // the default plan has the most parts (the variants' plans aim at fewer waves)
    const StreamPlan p = make_stream_plan(batch, L, dim, 4);
    return p.parts > 1 ? (size_t)p.groups * (p.parts - 1) * (N + 1) * stream::kLanes * 4 + 256 : 0;
}

namespace {

template <typename TIO>
hipError_t launch_default(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    const stream::ExtParams none = {nullptr, nullptr, 0, 0};
    switch (a.N) {
    case 4: return stream::launch_n<4, 0, TIO>(a, none, p, summ, s);
    case 8: return stream::launch_n<8, 0, TIO>(a, none, p, summ, s);
    case 16: return stream::launch_n<16, 0, TIO>(a, none, p, summ, s);
    case 32: return stream::launch_n<32, 0, TIO>(a, none, p, summ, s);
    case 64: return stream::launch_n<64, 0, TIO>(a, none, p, summ, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_fwd_stream(const FwdArgs &a, hipStream_t stream)
{
    const StreamPlan p = make_stream_plan(a.batch, a.L, a.dim);
    float *summ = stream::summary_buffer(a.workspace);
    return a.dtype == 1 ? launch_default<uint16_t>(a, p, summ, stream)
                        : launch_default<float>(a, p, summ, stream);
}

namespace {

template <int N, typename TIO>
hipError_t summaries_n(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    using namespace stream;
    const ExtParams none = {nullptr, nullptr, 0, 0};
    const int64_t waves = p.groups * (p.parts - 1);
    if (waves <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((fwd_stream_kernel<N, true, 0, TIO>),
                       dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kLanes * kWavesPerBlock), 0, s, (const TIO *)a.u,
                       (const TIO *)a.delta, (const TIO *)nullptr, (TIO *)nullptr, a.A,
                       (const TIO *)a.Bm, (const TIO *)a.Cm, (const float *)nullptr,
                       a.delta_bias, a.delta_softplus, (const float *)nullptr, (float *)nullptr,
                       summ, a.L, a.dim, p.groups, p.parts, p.part_len, none);
    return hipGetLastError();
}

template <typename TIO>
hipError_t summaries_t(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    switch (a.N) {
    case 4: return summaries_n<4, TIO>(a, p, summ, s);
    case 8: return summaries_n<8, TIO>(a, p, summ, s);
    case 16: return summaries_n<16, TIO>(a, p, summ, s);
    case 32: return summaries_n<32, TIO>(a, p, summ, s);
    case 64: return summaries_n<64, TIO>(a, p, summ, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_fwd_summaries(const FwdArgs &a, const StreamPlan &p, float *summ,
                                hipStream_t stream)
{
    return a.dtype == 1 ? summaries_t<uint16_t>(a, p, summ, stream)
                        : summaries_t<float>(a, p, summ, stream);
}

hipError_t launch_fwd_summaries_ext(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                   float *summ, hipStream_t stream)
{
    const bool zoh = (e.flags & kFwdFlagZohExact) != 0;
#define SELSCAN_EXT_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return zoh ? launch_fwd_summaries_ext_n##NN##_zoh(a, e, p, summ, stream)                  \
                   : launch_fwd_summaries_ext_n##NN(a, e, p, summ, stream);
    switch (a.N) {
    SELSCAN_EXT_CASE(4)
    SELSCAN_EXT_CASE(8)
    SELSCAN_EXT_CASE(16)
    SELSCAN_EXT_CASE(32)
    SELSCAN_EXT_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_EXT_CASE
}

hipError_t launch_fwd_stream_ext(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    const bool zoh = (e.flags & kFwdFlagZohExact) != 0;
#define SELSCAN_EXT_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return zoh ? launch_fwd_stream_ext_n##NN##_zoh(a, e, stream)                              \
                   : launch_fwd_stream_ext_n##NN(a, e, stream);
    switch (a.N) {
    SELSCAN_EXT_CASE(4)
    SELSCAN_EXT_CASE(8)
    SELSCAN_EXT_CASE(16)
    SELSCAN_EXT_CASE(32)
    SELSCAN_EXT_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_EXT_CASE
}

} // namespace selscan
