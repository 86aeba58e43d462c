// Variant instantiations of the streaming forward for state size N = 8 with
// B_bar = Delta B in the forward direction, direction and softplus switch
// fixed at compile time (launch_ext_fixed): the conv1d + SiLU prologue.
// A unit of its own so that it compiles in parallel with the
// reverse-direction variants of fwd_stream_ext_n8.hip.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {

template hipError_t launch_ext_fixed<8, false, uint16_t>(const FwdArgs &, const ExtParams &,
                                                     const StreamPlan &, float *, float *,
                                                     hipStream_t);
template hipError_t launch_ext_fixed<8, false, float>(const FwdArgs &, const ExtParams &,
                                                  const StreamPlan &, float *, float *,
                                                  hipStream_t);

} // namespace stream
} // namespace selscan
