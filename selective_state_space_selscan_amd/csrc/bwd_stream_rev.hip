// Backward of the selective scan, instantiated for the Euler B_bar in the
// reverse direction, fixed at compile time: the default's code with the
// addressing mirrored.  One translation unit per variant so that they compile
// in parallel; the kernels are in bwd_stream_impl.hpp.
#include "bwd_stream_impl.hpp"

namespace selscan {

hipError_t launch_bwd_euler_rev(const BwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return bwd::launch_bwd_var<stream::kVarRev>(a, e, stream);
}

} // namespace selscan
