// Variant instantiations of the streaming forward for state size N = 64 with
// exact zero-order hold B_bar in the forward direction, direction and softplus switch
// fixed at compile time (launch_ext_fixed): the conv1d + SiLU prologue, and the scan without it;
// fp32 I/O.  Apart from the bf16 ones (fwd_stream_ext_n64_zoh_fixed.hip) because
// together they were the build's slowest unit by far.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {

template hipError_t launch_ext_fixed<64, true, float>(const FwdArgs &, const ExtParams &,
                                                  const StreamPlan &, float *, float *,
                                                  hipStream_t);

} // namespace stream
} // namespace selscan
