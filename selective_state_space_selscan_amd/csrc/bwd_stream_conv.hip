// Backward of the selective scan, instantiated for the conv1d + SiLU prologue (Euler B_bar)
// (either direction).  One translation unit per variant so that they compile
// in parallel; the kernels are in bwd_stream_impl.hpp.
#include "bwd_stream_impl.hpp"

namespace selscan {

hipError_t launch_bwd_euler_conv(const BwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return bwd::launch_bwd_var<stream::kVarExt | stream::kVarConv>(a, e, stream);
}

} // namespace selscan
