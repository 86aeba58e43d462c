// Variant instantiations of the streaming forward for state size N = 64 with
// exact zero-order hold B_bar: the variants with REVERSE (the direction fixed
// at compile time) and the summary pass the variants' backward uses (the
// direction a run-time flag); the forward-direction variants are in the
// matching _fixed unit.  One
// translation unit per (N, B_bar form) so that they compile in parallel.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {
// compiled in fwd_stream_ext_n64_zoh_fixed.hip
extern template hipError_t launch_ext_fixed<64, true, uint16_t>(const FwdArgs &, const ExtParams &,
                                                            const StreamPlan &, float *, float *,
                                                            hipStream_t);
extern template hipError_t launch_ext_fixed<64, true, float>(const FwdArgs &, const ExtParams &,
                                                         const StreamPlan &, float *, float *,
                                                         hipStream_t);
// compiled in fwd_stream_ext_n64_zoh_rev_f32.hip: the reverse variants with
// fp32 I/O
extern template hipError_t launch_n<64, kVarRev | kVarZoh, float>(const FwdArgs &,
                                                                 const ExtParams &,
                                                                 const StreamPlan &, float *,
                                                                 float *, hipStream_t);
extern template hipError_t launch_n<64, kVarRev | kVarZoh | kVarConv, float>(
    const FwdArgs &, const ExtParams &, const StreamPlan &, float *, float *, hipStream_t);
} // namespace stream

hipError_t launch_fwd_stream_ext_n64_zoh(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return stream::launch_ext<64, true>(a, e, stream);
}

hipError_t launch_fwd_summaries_ext_n64_zoh(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                        float *summ, hipStream_t stream)
{
    return stream::launch_ext_summaries<64, true>(a, e, p, summ, stream);
}

} // namespace selscan
