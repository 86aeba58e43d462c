// Variant instantiations of the streaming forward for state size N = 32 with
// exact zero-order hold B_bar: reverse direction (run-time flag) and the conv1d + SiLU
// prologue.  One translation unit per (N, B_bar form) so that they compile in
// parallel.
#include "fwd_stream_impl.hpp"

namespace selscan {

hipError_t launch_fwd_stream_ext_n32_zoh(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return stream::launch_ext<32, true>(a, e, stream);
}

hipError_t launch_fwd_summaries_ext_n32_zoh(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                        float *summ, hipStream_t stream)
{
    return stream::launch_ext_summaries<32, true>(a, e, p, summ, stream);
}

} // namespace selscan
