// The default forward (or the reverse-alone one) whose main pass also keeps
// the backward's checkpoints:
// the state entering every 4-step chunk, stored where a backward that reuses
// this workspace (SELSCAN_FLAG_REUSE_FWD_STATE with
// SELSCAN_FLAG_KEEP_CHECKPOINTS) reads them instead of recomputing them in its
// checkpoint pass.  The paper walkthrough (m.lqnn.cn) §3.4 has the forward
// keep only its inputs and the backward recompute the states; its §5.4 leaves
// that trade to the user (with memory to spare, recompute less for speed).
// This keeps one state in four (16 B per element at N = 16) for the
// backward's walk over the sequence.  A translation unit of its own (the main
// pass instantiated with kVarKeep), compiled in parallel with the others.
#include "fwd_stream_impl.hpp"

namespace selscan {

namespace {

template <int V, typename TIO>
hipError_t launch_keep(const FwdArgs &a, const StreamPlan &p, float *summ, float *entry,
                       const stream::ExtParams &x, hipStream_t s)
{
    switch (a.N) {
    case 4: return stream::launch_n<4, V, TIO>(a, x, p, summ, entry, s);
    case 8: return stream::launch_n<8, V, TIO>(a, x, p, summ, entry, s);
    case 16: return stream::launch_n<16, V, TIO>(a, x, p, summ, entry, s);
    case 32: return stream::launch_n<32, V, TIO>(a, x, p, summ, entry, s);
    case 64: return stream::launch_n<64, V, TIO>(a, x, p, summ, entry, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_fwd_stream_keep(const FwdArgs &a, bool reverse, hipStream_t stream)
{
    const StreamPlan p = default_fwd_plan(a.batch, a.L, a.dim);
    float *summ = stream::summary_buffer(a.workspace);   // the workspace aligned to 256 B
    float *entry = stream::entry_buffer(a.workspace, p, a.N);
    stream::ExtParams x{};
    x.ckpt = (float *)((char *)summ + bwd_checkpoint_offset(a.batch, a.L, a.dim, a.N));
    x.nck = (a.L + stream::TT - 1) / stream::TT;
    x.rev = reverse ? 1 : 0;
    if (reverse) {
        // the reverse-alone forward's code (kVarRev), checkpoints in scan order
        constexpr int V = stream::kVarKeep | stream::kVarRev;
        return a.dtype == 1 ? launch_keep<V, uint16_t>(a, p, summ, entry, x, stream)
                            : launch_keep<V, float>(a, p, summ, entry, x, stream);
    }
    constexpr int V = stream::kVarKeep;
    return a.dtype == 1 ? launch_keep<V, uint16_t>(a, p, summ, entry, x, stream)
                        : launch_keep<V, float>(a, p, summ, entry, x, stream);
}

} // namespace selscan
