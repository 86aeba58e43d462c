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

// Chunked forward (ablation: wave segments of a chunk exchange their
// aggregates through LDS): workspace bytes it needs, and the launch.
size_t fwd_chunked_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_chunked(const FwdArgs &a, hipStream_t stream);

// Forward with an in-wave DPP scan over time (ablation: lanes are the 64
// steps of a tile of one channel): workspace bytes it needs, and the launch.
size_t fwd_dpp_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_dpp(const FwdArgs &a, hipStream_t stream);

// Streaming forward (default): independent waves over sequence parts, with a
// summary pre-pass when the sequence is split.
constexpr int kStreamTT = 4;   // part lengths are multiples of this many steps
struct StreamPlan {
    int64_t groups;     // batch * ceil(dim / 64) channel groups
    int64_t part_len;   // steps per sequence part
    int parts;
};
// waves_per_simd: the kernel's occupancy; the plan aims at waves_per_slot_x2 / 2
// waves per wave slot of the chip; max_part_len (0: none) caps the length of a
// part.
StreamPlan make_stream_plan(int64_t batch, int64_t L, int64_t dim, int waves_per_simd = 4,
                            int waves_per_slot_x2 = 2, int64_t max_part_len = 0);
// The plan of the default forward (and of the reverse-alone variant, which
// runs the same code): one wave per slot at four waves per SIMD, parts of at
// most kDefaultFwdMaxPartLen steps.
constexpr int64_t kDefaultFwdMaxPartLen = 416;
StreamPlan default_fwd_plan(int64_t batch, int64_t L, int64_t dim);
size_t fwd_stream_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_stream(const FwdArgs &a, hipStream_t stream);

// Single-pass streaming forward with decoupled look-back (same plan).
// spin_limit: polls before a wait gives up (< 0: the default).  Word
// kLookbackStatusWord of the aligned workspace is nonzero after a call in
// which some wait gave up.
constexpr int kLookbackStatusWord = 1;
constexpr int kLookbackFlagsOffset = 2;   // words: ticket, status, then the flags
size_t fwd_lookback_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
hipError_t launch_fwd_lookback(const FwdArgs &a, int spin_limit, hipStream_t stream);

// Variants of the streaming forward (same plan and workspace).
constexpr int kFwdFlagZohExact = 1;
constexpr int kFwdFlagReverse = 2;
constexpr int kBwdFlagReuseFwdState = 4;   // backward: the workspace holds the forward's part state
// forward: the main pass also stores the backward's checkpoints (the state
// entering every 4-step chunk) in the workspace, at the backward layout's
// offset; backward (with kBwdFlagReuseFwdState): they are there.
constexpr int kFwdFlagKeepCheckpoints = 8;
struct FwdExt {
    int flags;            // kFwdFlagZohExact | kFwdFlagReverse
    const float *conv_w;  // (dim, conv_k) when conv_k > 0
    const float *conv_b;  // (dim) or null
    int conv_k;           // 0 = no conv prologue, else 1..4
};
hipError_t launch_fwd_stream_ext(const FwdArgs &a, const FwdExt &e, hipStream_t stream);
// The default forward (reverse: the reverse-alone one) with
// kFwdFlagKeepCheckpoints (fwd_stream_keep.hip); its workspace is a
// backward's (bwd_workspace_bytes).
hipError_t launch_fwd_stream_keep(const FwdArgs &a, bool reverse, hipStream_t stream);
// Byte offset of the checkpoint buffer in the backward's workspace layout,
// from the workspace aligned up to 256 bytes.
size_t bwd_checkpoint_offset(int64_t batch, int64_t L, int64_t dim, int64_t N);
// One translation unit per (N, B_bar form): fwd_stream_ext_n<N>[_zoh].hip.
#define SELSCAN_DECLARE_EXT(NN)                                                                   \
    hipError_t launch_fwd_stream_ext_n##NN(const FwdArgs &a, const FwdExt &e, hipStream_t s);    \
    hipError_t launch_fwd_stream_ext_n##NN##_zoh(const FwdArgs &a, const FwdExt &e, hipStream_t s); \
    hipError_t launch_fwd_summaries_ext_n##NN(const FwdArgs &a, const FwdExt &e,                 \
                                              const StreamPlan &p, float *summ, hipStream_t s);  \
    hipError_t launch_fwd_summaries_ext_n##NN##_zoh(const FwdArgs &a, const FwdExt &e,           \
                                                    const StreamPlan &p, float *summ, hipStream_t s);
SELSCAN_DECLARE_EXT(4)
SELSCAN_DECLARE_EXT(8)
SELSCAN_DECLARE_EXT(16)
SELSCAN_DECLARE_EXT(32)
SELSCAN_DECLARE_EXT(64)
#undef SELSCAN_DECLARE_EXT

// Entry states of the parts from the part summaries (groups, P - 1, N + 1, 64)
// into entry (groups, P, N, 64): h0 (init, or 0) folded through the summaries
// of the earlier parts; with reverse = 1, from the right (the backward's
// adjoint, init = dh_last).
// scratch: carry_scratch_bytes(groups, parts, N) bytes for the two-level carry
// of many parts (null: the single-level carry).
hipError_t launch_fwd_carry(const float *summ, const float *init, const float *A, float *entry,
                            int64_t batch, int64_t dim, int64_t N, int parts, int reverse,
                            float *scratch, hipStream_t stream);
size_t carry_scratch_bytes(int64_t groups, int parts, int64_t N);

// Forward part summaries alone (the summary pass of the streaming forward,
// default instantiation) into summ: (groups, parts - 1, N + 1, 64) fp32.
hipError_t launch_fwd_summaries(const FwdArgs &a, const StreamPlan &p, float *summ,
                                hipStream_t stream);
// The same for a variant forward.
hipError_t launch_fwd_summaries_ext(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                   float *summ, hipStream_t stream);

// Backward (gradients of the default forward, or of a variant forward).
// `fwd` carries the forward's inputs, dtype, sizes and the workspace; its y
// and h_last are unused.
struct BwdArgs {
    FwdArgs fwd;
    const void *dy;         // (batch, L, dim) dtype
    const float *dh_last;   // (batch, dim, N) or null
    void *du, *ddelta, *dz; // (batch, L, dim) dtype; dz only with z
    float *dA;              // (dim, N)
    float *dB, *dC;         // (batch, L, N)
    float *dD, *ddelta_bias;// (dim) or null
    float *dh0;             // (batch, dim, N) or null
    float *dconv_w;         // (dim, conv_k): with the conv prologue only
    float *dconv_b;         // (dim) or null: with the conv prologue only
};
size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
// e: the variant (null or flags 0 without conv: the default forward).
hipError_t launch_bwd(const BwdArgs &a, const FwdExt *e, hipStream_t stream);
// One translation unit per variant: bwd_stream[_rev|_zoh|_conv|_zoh_conv].hip.
hipError_t launch_bwd_euler(const BwdArgs &a, const FwdExt &e, hipStream_t stream);
hipError_t launch_bwd_euler_rev(const BwdArgs &a, const FwdExt &e, hipStream_t stream);
hipError_t launch_bwd_zoh(const BwdArgs &a, const FwdExt &e, hipStream_t stream);
hipError_t launch_bwd_euler_conv(const BwdArgs &a, const FwdExt &e, hipStream_t stream);
hipError_t launch_bwd_zoh_conv(const BwdArgs &a, const FwdExt &e, hipStream_t stream);

// Decode step.
hipError_t launch_state_update(const StepArgs &a, hipStream_t stream);

} // namespace selscan
