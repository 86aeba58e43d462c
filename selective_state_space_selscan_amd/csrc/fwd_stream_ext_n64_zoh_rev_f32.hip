// Variant instantiations of the streaming forward for state size N = 64 with
// exact zero-order hold B_bar in reverse, direction fixed at compile time, with
// and without the conv1d + SiLU prologue; fp32 I/O.  Apart from the bf16 ones
// (fwd_stream_ext_n64_zoh.hip) so that the two compile in parallel: together
// they made the build's slowest unit.
#include "fwd_stream_impl.hpp"

namespace selscan {
namespace stream {

template hipError_t launch_n<64, kVarRev | kVarZoh, float>(const FwdArgs &, const ExtParams &,
                                                          const StreamPlan &, float *, float *,
                                                          hipStream_t);
template hipError_t launch_n<64, kVarRev | kVarZoh | kVarConv, float>(
    const FwdArgs &, const ExtParams &, const StreamPlan &, float *, float *, hipStream_t);

} // namespace stream
} // namespace selscan
