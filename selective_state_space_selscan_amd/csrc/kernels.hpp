// Internal launch interface between the C-ABI layer (selscan_api.hip) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace selscan {

struct FwdArgs {
    const void *u;
    const void *delta;
    const float *A;
    const void *Bm;
    const void *Cm;
    const float *D_skip;
    const void *z;
    const float *delta_bias;
    int delta_softplus;
    const float *h0;
    void *y;
    float *h_last;
    int64_t batch, L, dim, N;
    int dtype;              // 0 = fp32, 1 = bf16
    void *workspace;
    size_t workspace_bytes;
};

struct StepArgs {
    float *state;
    const void *u;
    const void *delta;
    const float *A;
    const void *Bm;
    const void *Cm;
    const float *D_skip;
    const void *z;
    const float *delta_bias;
    int delta_softplus;
    void *y;
    int64_t batch, dim, N;
    int dtype;
};

// Serial forward: one lane per (batch, channel), whole sequence in-lane.
hipError_t launch_fwd_serial(const FwdArgs &a, hipStream_t stream);

// Chunked forward (the fast path): workspace bytes it needs, and the launch.
size_t fwd_chunked_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_chunked(const FwdArgs &a, hipStream_t stream);

// Streaming forward (default): independent waves over sequence parts, with a
// summary pre-pass when the sequence is split.
size_t fwd_stream_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_stream(const FwdArgs &a, hipStream_t stream);

// Decode step.
hipError_t launch_state_update(const StepArgs &a, hipStream_t stream);

} // namespace selscan
