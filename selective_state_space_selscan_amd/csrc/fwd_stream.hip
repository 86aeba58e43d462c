// Streaming selective-scan forward: launch plan, the default instantiation
// (Euler B_bar = Delta B, forward direction, no prologue) and the dispatch of
// the variants.  The kernel itself is in fwd_stream_impl.hpp.
#include "fwd_stream_impl.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace selscan {

// SELSCAN_STREAM_PARTS=P overrides the number of sequence parts (tuning knob).
// Default (measured on MI355X with the clocks ramped up): waves_per_slot_x2 / 2
// waves per wave slot of the chip (1024 SIMDs x the kernel's waves per SIMD)
// when the channel groups are few; with many groups, at least 8 parts (when L
// allows), since smaller waves balance the tail of the grid better than fewer,
// longer ones, and for the same reason on a long sequence parts of at most
// max_part_len steps.  The default forward: one wave per slot, parts of at
// most 416 steps: mamba130m_layer 22 parts of 96 steps (1.5 % faster than 32
// of 64), long_seq 316 parts of 416 (2.7 % faster than 192 of 684),
// large_layer 8 parts of 256.  Parts are whole multiples of kStreamTT steps
// and at least 4 of them long.
StreamPlan make_stream_plan(int64_t batch, int64_t L, int64_t dim, int waves_per_simd,
                            int waves_per_slot_x2, int64_t max_part_len)
{
    constexpr int kLanes = stream::kLanes;
    constexpr int TT = kStreamTT;
    StreamPlan p;
    p.groups = batch * ((dim + kLanes - 1) / kLanes);
    const int64_t target_waves = 512 * (int64_t)waves_per_simd * waves_per_slot_x2;
    int64_t parts = (target_waves + p.groups - 1) / p.groups;
    int64_t min_parts = L / 256 < 8 ? L / 256 : 8;
    if (max_part_len > 0 && (L + max_part_len - 1) / max_part_len > min_parts)
        min_parts = (L + max_part_len - 1) / max_part_len;
    if (parts < min_parts)
        parts = min_parts;
    const char *e = getenv("SELSCAN_STREAM_PARTS");
    long long ov = 0;
    if (e && sscanf(e, "%lld", &ov) == 1 && ov >= 1)
        parts = ov;
    const int64_t max_parts = (L + 4 * TT - 1) / (4 * TT);
    if (parts > max_parts)
        parts = max_parts;
    if (parts > 65536)
        parts = 65536;
    if (parts < 1)
        parts = 1;
    p.part_len = (L + parts - 1) / parts;
    p.part_len = (p.part_len + TT - 1) / TT * TT;
    p.parts = (int)((L + p.part_len - 1) / p.part_len);
    return p;
}

StreamPlan default_fwd_plan(int64_t batch, int64_t L, int64_t dim)
{
    return make_stream_plan(batch, L, dim, 4, 2, kDefaultFwdMaxPartLen);
}

size_t fwd_stream_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    // the default forward's plan has the most parts (the other plans aim at
    // fewer waves): the part summaries, then the entry states of the parts
    const StreamPlan p = default_fwd_plan(batch, L, dim);
    if (p.parts <= 1)
        return 0;
    const size_t summ = (size_t)p.groups * (p.parts - 1) * (N + 1) * stream::kLanes * 4;
    const size_t entry = (size_t)p.groups * p.parts * N * stream::kLanes * 4;
    return 256 + ((summ + 255) & ~(size_t)255) + ((entry + 255) & ~(size_t)255) +
           carry_scratch_bytes(p.groups, p.parts, N);
}

namespace {

// Entry states of the parts from the part summaries: the exclusive prefix of
// the associative fold h <- exp(A S) h + x (S the part's sum of Delta, x its
// end state from zero).  One lane per (channel group, state n, channel): the
// fold runs over the parts in sequence, its loads kCarryBatch parts ahead.
//   forward (reverse = 0): entry[0] = init (h0, or 0), and entry[j + 1] =
//     summary j folded into entry[j];
//   reverse (reverse = 1, the backward's adjoint): entry[P-1] = init
//     (dh_last, or 0), and entry[j] = summary j (that of part j + 1) folded
//     into entry[j + 1].
// summ: (groups, P - 1, N + 1, 64); entry: (groups, P, N, 64); init:
// (batch, dim, N) or null.
constexpr int kCarryBatch = 16;

template <int N>
__global__ __launch_bounds__(256) void carry_kernel(const float *__restrict__ summ,
                                                    const float *__restrict__ init,
                                                    const float *__restrict__ A,
                                                    float *__restrict__ entry, int64_t dim,
                                                    int64_t groups, int parts, int reverse)
{
    constexpr int kLanes = stream::kLanes;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = (int)(tid & (kLanes - 1));
    const int64_t wn = tid / kLanes;   // (group, n), wave-uniform
    if (wn >= groups * N)
        return;
    const int n = (int)(wn % N);
    const int64_t grp = wn / N;
    const int64_t gpr = (dim + kLanes - 1) / kLanes;
    const int64_t b = grp / gpr;
    const int64_t d0 = (grp % gpr) * kLanes;
    const int64_t d = d0 + lane < dim ? d0 + lane : dim - 1;
    const float a2 = A[d * N + n] * kLog2e;
    float h = init ? init[(b * dim + d) * N + n] : 0.0f;
    const int64_t sstride = (int64_t)(N + 1) * kLanes;   // between summaries
    const int64_t estride = (int64_t)N * kLanes;         // between entry states
    const float *sb = summ + grp * (parts - 1) * sstride + lane;
    float *eb = entry + grp * parts * estride + n * kLanes + lane;
    const int J = parts - 1;
    eb[(reverse ? J : 0) * estride] = h;
    for (int k0 = 0; k0 < J; k0 += kCarryBatch) {
        float S[kCarryBatch], X[kCarryBatch];
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            const int j = reverse ? J - 1 - (k0 + k) : k0 + k;
            const bool in = k0 + k < J;
            S[k] = in ? sb[j * sstride] : 0.0f;
            X[k] = in ? sb[j * sstride + (n + 1) * kLanes] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (k0 + k < J) {
                const int j = reverse ? J - 1 - (k0 + k) : k0 + k;
                h = fmaf(hw_exp2(a2 * S[k]), h, X[k]);
                eb[(reverse ? j : j + 1) * estride] = h;
            }
        }
    }
}

// Two-level carry for many parts: the summaries are taken in blocks of
// kCarryBlock; the blocks' aggregates (decay sum and end state from zero, the
// summary of the whole block) are folded by carry_kernel, and each block's
// entries then filled from its carried start.  The sequential depth drops
// from P to about 2 kCarryBlock + P / kCarryBlock.
constexpr int kCarryBlock = 64;

__host__ __device__ inline int64_t carry_blocks(int parts)
{
    return (parts - 1 + kCarryBlock - 1) / kCarryBlock;
}

// fill = false: the aggregate of block blk into bsumm (groups, nb, N + 1, 64),
// in the fold's order (from the right with reverse).  fill = true: the block's
// entries, folded from bentry (groups, nb + 1, N, 64, from carry_kernel) into
// entry.  One lane per (group, block, n, channel).
template <int N>
__global__ __launch_bounds__(256) void carry_block_kernel(const float *__restrict__ summ,
                                                          const float *__restrict__ A,
                                                          float *__restrict__ bsumm,
                                                          const float *__restrict__ bentry,
                                                          float *__restrict__ entry,
                                                          const float *__restrict__ init,
                                                          int64_t dim, int64_t groups, int parts,
                                                          int reverse, int fill)
{
    constexpr int kLanes = stream::kLanes;
    const int64_t nb = carry_blocks(parts);
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = (int)(tid & (kLanes - 1));
    int64_t w = tid / kLanes;   // (group, block, n), wave-uniform
    if (w >= groups * nb * N)
        return;
    const int n = (int)(w % N);
    w /= N;
    const int64_t blk = w % nb;
    const int64_t grp = w / nb;
    const int64_t gpr = (dim + kLanes - 1) / kLanes;
    const int64_t d0 = (grp % gpr) * kLanes;
    const int64_t d = d0 + lane < dim ? d0 + lane : dim - 1;
    const float a2 = A[d * N + n] * kLog2e;
    const int J = parts - 1;
    const int j_lo = (int)(blk * kCarryBlock);
    const int j_hi = j_lo + kCarryBlock < J ? j_lo + kCarryBlock : J;
    const int cnt = j_hi - j_lo;
    const int64_t sstride = (int64_t)(N + 1) * kLanes;
    const int64_t estride = (int64_t)N * kLanes;
    const float *sb = summ + grp * (parts - 1) * sstride + lane;
    float *eb = entry + grp * parts * estride + n * kLanes + lane;
    const float *be = bentry + (grp * (nb + 1)) * estride + n * kLanes + lane;
    float h = 0.0f, S = 0.0f;
    if (fill) {
        // state before the block: from the left E[j_lo], from the right E[j_hi]
        h = be[(reverse ? blk + 1 : blk) * estride];
        if (!reverse && blk == 0)
            eb[0] = h;
        if (reverse && blk == nb - 1)
            eb[(int64_t)J * estride] = h;
    }
    for (int k0 = 0; k0 < cnt; k0 += kCarryBatch) {
        float Sv[kCarryBatch], X[kCarryBatch];
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            const int j = reverse ? j_hi - 1 - (k0 + k) : j_lo + k0 + k;
            const bool in = k0 + k < cnt;
            Sv[k] = in ? sb[j * sstride] : 0.0f;
            X[k] = in ? sb[j * sstride + (n + 1) * kLanes] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kCarryBatch; ++k) {
            if (k0 + k < cnt) {
                const int j = reverse ? j_hi - 1 - (k0 + k) : j_lo + k0 + k;
                h = fmaf(hw_exp2(a2 * Sv[k]), h, X[k]);
                S += Sv[k];
                if (fill)
                    eb[(reverse ? j : j + 1) * estride] = h;
            }
        }
    }
    if (!fill) {
        float *o = bsumm + (grp * nb + blk) * sstride + lane;
        if (n == 0)
            o[0] = S;
        o[(n + 1) * kLanes] = h;
    }
    (void)init;
}

template <int N>
hipError_t carry_n(const float *summ, const float *init, const float *A, float *entry,
                   int64_t batch, int64_t dim, int parts, int reverse, float *scratch,
                   hipStream_t s)
{
    const int64_t groups = batch * ((dim + stream::kLanes - 1) / stream::kLanes);
    const int64_t nb = carry_blocks(parts);
    if (!scratch || nb <= 2) {
        const int64_t threads = groups * N * stream::kLanes;
        hipLaunchKernelGGL((carry_kernel<N>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, s, summ, init, A, entry, dim, groups, parts, reverse);
        return hipGetLastError();
    }
    float *bsumm = scratch;
    float *bentry = scratch + groups * nb * (N + 1) * stream::kLanes;
    const int64_t threads = groups * nb * N * stream::kLanes;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    hipLaunchKernelGGL((carry_block_kernel<N>), grid, block, 0, s, summ, A, bsumm,
                       (const float *)nullptr, entry, init, dim, groups, parts, reverse, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t t2 = groups * N * stream::kLanes;
    hipLaunchKernelGGL((carry_kernel<N>), dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, s,
                       (const float *)bsumm, init, A, bentry, dim, groups, (int)nb + 1, reverse);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL((carry_block_kernel<N>), grid, block, 0, s, summ, A, (float *)nullptr,
                       (const float *)bentry, entry, init, dim, groups, parts, reverse, 1);
    return hipGetLastError();
}

} // namespace

size_t carry_scratch_bytes(int64_t groups, int parts, int64_t N)
{
    const int64_t nb = carry_blocks(parts);
    if (parts <= 1 || nb <= 2)
        return 0;
    return (size_t)groups * (nb * (N + 1) + (nb + 1) * N) * stream::kLanes * 4;
}

hipError_t launch_fwd_carry(const float *summ, const float *init, const float *A, float *entry,
                            int64_t batch, int64_t dim, int64_t N, int parts, int reverse,
                            float *scratch, hipStream_t stream)
{
    switch (N) {
    case 4: return carry_n<4>(summ, init, A, entry, batch, dim, parts, reverse, scratch, stream);
    case 8: return carry_n<8>(summ, init, A, entry, batch, dim, parts, reverse, scratch, stream);
    case 16: return carry_n<16>(summ, init, A, entry, batch, dim, parts, reverse, scratch, stream);
    case 32: return carry_n<32>(summ, init, A, entry, batch, dim, parts, reverse, scratch, stream);
    case 64: return carry_n<64>(summ, init, A, entry, batch, dim, parts, reverse, scratch, stream);
    default: return hipErrorInvalidValue;
    }
}

namespace {

template <typename TIO>
hipError_t launch_default(const FwdArgs &a, const StreamPlan &p, float *summ, float *entry,
                          hipStream_t s)
{
    const stream::ExtParams none = {nullptr, nullptr, 0, 0};
    switch (a.N) {
    case 4: return stream::launch_n<4, 0, TIO>(a, none, p, summ, entry, s);
    case 8: return stream::launch_n<8, 0, TIO>(a, none, p, summ, entry, s);
    case 16: return stream::launch_n<16, 0, TIO>(a, none, p, summ, entry, s);
    case 32: return stream::launch_n<32, 0, TIO>(a, none, p, summ, entry, s);
    case 64: return stream::launch_n<64, 0, TIO>(a, none, p, summ, entry, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_fwd_stream(const FwdArgs &a, hipStream_t stream)
{
    const StreamPlan p = default_fwd_plan(a.batch, a.L, a.dim);
    float *summ = stream::summary_buffer(a.workspace);
    float *entry = stream::entry_buffer(a.workspace, p, a.N);
    return a.dtype == 1 ? launch_default<uint16_t>(a, p, summ, entry, stream)
                        : launch_default<float>(a, p, summ, entry, stream);
}

namespace {

template <int N, typename TIO>
hipError_t summaries_n(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    using namespace stream;
    const ExtParams none = {nullptr, nullptr, 0, 0};
    const int64_t waves = p.groups * (p.parts - 1);
    if (waves <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((fwd_stream_kernel<N, true, 0, TIO>),
                       dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kLanes * kWavesPerBlock), 0, s, (const TIO *)a.u,
                       (const TIO *)a.delta, (const TIO *)nullptr, (TIO *)nullptr, a.A,
                       (const TIO *)a.Bm, (const TIO *)a.Cm, (const float *)nullptr,
                       a.delta_bias, a.delta_softplus, (const float *)nullptr, (float *)nullptr,
                       summ, (const float *)nullptr, a.L, a.dim, p.groups, p.parts, p.part_len,
                       none);
    return hipGetLastError();
}

template <typename TIO>
hipError_t summaries_t(const FwdArgs &a, const StreamPlan &p, float *summ, hipStream_t s)
{
    switch (a.N) {
    case 4: return summaries_n<4, TIO>(a, p, summ, s);
    case 8: return summaries_n<8, TIO>(a, p, summ, s);
    case 16: return summaries_n<16, TIO>(a, p, summ, s);
    case 32: return summaries_n<32, TIO>(a, p, summ, s);
    case 64: return summaries_n<64, TIO>(a, p, summ, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_fwd_summaries(const FwdArgs &a, const StreamPlan &p, float *summ,
                                hipStream_t stream)
{
    return a.dtype == 1 ? summaries_t<uint16_t>(a, p, summ, stream)
                        : summaries_t<float>(a, p, summ, stream);
}

hipError_t launch_fwd_summaries_ext(const FwdArgs &a, const FwdExt &e, const StreamPlan &p,
                                   float *summ, hipStream_t stream)
{
    const bool zoh = (e.flags & kFwdFlagZohExact) != 0;
#define SELSCAN_EXT_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return zoh ? launch_fwd_summaries_ext_n##NN##_zoh(a, e, p, summ, stream)                  \
                   : launch_fwd_summaries_ext_n##NN(a, e, p, summ, stream);
    switch (a.N) {
    SELSCAN_EXT_CASE(4)
    SELSCAN_EXT_CASE(8)
    SELSCAN_EXT_CASE(16)
    SELSCAN_EXT_CASE(32)
    SELSCAN_EXT_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_EXT_CASE
}

hipError_t launch_fwd_stream_ext(const FwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    // the backward's checkpoints kept: the plain forward or reverse alone
    if ((e.flags & kFwdFlagKeepCheckpoints) != 0 && e.conv_k == 0 &&
        (e.flags & ~(kFwdFlagKeepCheckpoints | kFwdFlagReverse)) == 0)
        return launch_fwd_stream_keep(a, (e.flags & kFwdFlagReverse) != 0, stream);
    // no variant: the default forward itself (same plan, same bits)
    if (e.flags == 0 && e.conv_k == 0)
        return launch_fwd_stream(a, stream);
    const bool zoh = (e.flags & kFwdFlagZohExact) != 0;
#define SELSCAN_EXT_CASE(NN)                                                                      \
    case NN:                                                                                      \
        return zoh ? launch_fwd_stream_ext_n##NN##_zoh(a, e, stream)                              \
                   : launch_fwd_stream_ext_n##NN(a, e, stream);
    switch (a.N) {
    SELSCAN_EXT_CASE(4)
    SELSCAN_EXT_CASE(8)
    SELSCAN_EXT_CASE(16)
    SELSCAN_EXT_CASE(32)
    SELSCAN_EXT_CASE(64)
    default: return hipErrorInvalidValue;
    }
#undef SELSCAN_EXT_CASE
}

} // namespace selscan
