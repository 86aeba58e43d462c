// Variant instantiations of the streaming forward for state size N = 32 with
// exact zero-order hold B_bar in the forward direction, direction and softplus switch
// fixed at compile time (launch_ext_fixed): the conv1d + SiLU prologue, and the scan without it.
// A unit of its own so that it compiles in parallel with the
// run-time-direction variants of fwd_stream_ext_n32_zoh.hip.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {

template hipError_t launch_ext_fixed<32, true, uint16_t>(const FwdArgs &, const ExtParams &,
                                                     const StreamPlan &, float *, float *,
                                                     hipStream_t);
template hipError_t launch_ext_fixed<32, true, float>(const FwdArgs &, const ExtParams &,
                                                  const StreamPlan &, float *, float *,
                                                  hipStream_t);

} // namespace stream
} // namespace selscan
