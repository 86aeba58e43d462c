// Variant instantiations of the streaming forward for state size N = 32 with
// B_bar = Delta B: the variants with REVERSE (the direction a run-time
// flag), reverse alone, and the summary pass the variants' backward uses; the
// forward-direction variants are in the matching _fixed unit.  One
// translation unit per (N, B_bar form) so that they compile in parallel.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {
// compiled in fwd_stream_ext_n32_fixed.hip
extern template hipError_t launch_ext_fixed<32, false, uint16_t>(const FwdArgs &, const ExtParams &,
                                                            const StreamPlan &, float *, float *,
                                                            hipStream_t);
extern template hipError_t launch_ext_fixed<32, false, float>(const FwdArgs &, const ExtParams &,
                                                         const StreamPlan &, float *, float *,
                                                         hipStream_t);
} // namespace stream

hipError_t launch_fwd_stream_ext_n32(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return stream::launch_ext<32, false>(a, e, stream);
}

hipError_t launch_fwd_summaries_ext_n32(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                        float *summ, hipStream_t stream)
{
    return stream::launch_ext_summaries<32, false>(a, e, p, summ, stream);
}

} // namespace selscan
