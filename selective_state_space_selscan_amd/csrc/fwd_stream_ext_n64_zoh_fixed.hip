// Variant instantiations of the streaming forward for state size N = 64 with
// exact zero-order hold B_bar in the forward direction, direction and softplus switch
// fixed at compile time (launch_ext_fixed): the conv1d + SiLU prologue, and the scan without it;
// bf16 I/O (fp32 I/O: fwd_stream_ext_n64_zoh_fixed_f32.hip).
// A unit of its own so that it compiles in parallel with the
// reverse-direction variants of fwd_stream_ext_n64_zoh.hip.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {

template hipError_t launch_ext_fixed<64, true, uint16_t>(const FwdArgs &, const ExtParams &,
                                                     const StreamPlan &, float *, float *,
                                                     hipStream_t);

} // namespace stream
} // namespace selscan
