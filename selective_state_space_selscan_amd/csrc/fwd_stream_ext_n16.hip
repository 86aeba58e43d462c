// Variant instantiations of the streaming forward for state size N = 16 with
// B_bar = Delta B: reverse direction (run-time flag) and the conv1d + SiLU
// prologue.  One translation unit per (N, B_bar form) so that they compile in
// parallel.
#include "fwd_stream_impl.hpp"

namespace selscan {

hipError_t launch_fwd_stream_ext_n16(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return stream::launch_ext<16, false>(a, e, stream);
}

hipError_t launch_fwd_summaries_ext_n16(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                        float *summ, hipStream_t stream)
{
    return stream::launch_ext_summaries<16, false>(a, e, p, summ, stream);
}

} // namespace selscan
