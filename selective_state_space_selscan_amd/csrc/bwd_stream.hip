// Backward of the selective scan: the reductions of the partials, the
// workspace layout, the dispatch over the variants and the instantiation for
// the Euler B_bar in the forward direction.  The kernels are in
// bwd_stream_impl.hpp.
#include "bwd_stream_impl.hpp"

namespace selscan {
namespace bwd {

// The column sums of all the partials of one backward call in one launch:
// for each job, out[i] = sum_k in[k * P + i] for i < P, k < K.  A block of 16
// waves owns 16 / S groups of 64 columns of one job; the S waves of a group
// add the rows k = s, s + S, ... (eight loads in flight), then their S sums
// are added in wave order, so the result does not depend on timing.  S grows
// with K (1, 4 or 16): the long, narrow reductions (dD, dbias over every
// wave's partial) are split over more waves, the short, wide ones (dB, dC
// over the channel groups) not at all.  The jobs' blocks follow each other
// in the grid, so the small, latency-bound jobs run beside the large ones.
constexpr int kColsumWaves = 16;

__host__ __device__ inline int colsum_split(int64_t K)
{
    return K >= 128 ? 16 : K >= 32 ? 4 : 1;
}

__global__ __launch_bounds__(kLanes * kColsumWaves) void bwd_colsum_kernel(ColsumJobs jobs)
{
    __shared__ float part[kColsumWaves][kLanes];
    const int lane = threadIdx.x & (kLanes - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // this block's job (fields read at constant offsets: no dynamic indexing
    // of the argument block)
    const int64_t blk = blockIdx.x;
    const float *in = jobs.j[0].in;
    float *out = jobs.j[0].out;
    int64_t P = jobs.j[0].P, K = jobs.j[0].K, b0 = 0;
#pragma unroll
    for (int q = 1; q < kMaxColsumJobs; ++q) {
        if (q < jobs.n && blk >= jobs.j[q].block0) {
            in = jobs.j[q].in;
            out = jobs.j[q].out;
            P = jobs.j[q].P;
            K = jobs.j[q].K;
            b0 = jobs.j[q].block0;
        }
    }
    const int S = colsum_split(K);
    const int grp = wave / S, sl = wave % S;
    const int64_t i = ((blk - b0) * (kColsumWaves / S) + grp) * kLanes + lane;
    float s = 0.0f;
    if (i < P) {
        int64_t k = sl;
        for (; k + 7 * S < K; k += 8 * S) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = in[(k + S * j) * P + i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s += v[j];
        }
        for (; k < K; k += S)
            s += in[k * P + i];
    }
    part[wave][lane] = s;
    __syncthreads();
    if (sl == 0 && i < P) {
        float t = part[wave][lane];
        for (int w = 1; w < S; ++w)
            t += part[wave + w][lane];
        out[i] = t;
    }
}

void ColsumJobs::add(const float *in, float *out, int64_t P, int64_t K)
{
    if (!out)
        return;   // an optional gradient the caller does not want (NULL = skip)
    if (n >= kMaxColsumJobs) {
        n = kMaxColsumJobs + 1;   // the table is full: launch_colsums refuses it
        return;
    }
    ColsumJob &c = j[n++];
    c.in = in;
    c.out = out;
    c.P = P;
    c.K = K;
    c.block0 = blocks;
    const int64_t cols = (int64_t)kLanes * (kColsumWaves / colsum_split(K));
    blocks += (P + cols - 1) / cols;
}

hipError_t launch_colsums(const ColsumJobs &jobs, hipStream_t s)
{
    if (jobs.n > kMaxColsumJobs || jobs.blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    for (int q = 0; q < jobs.n; ++q)
        if (!jobs.j[q].in || !jobs.j[q].out || jobs.j[q].P <= 0 || jobs.j[q].K <= 0)
            return hipErrorInvalidValue;
    if (jobs.n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(bwd_colsum_kernel, dim3((unsigned)jobs.blocks),
                       dim3(kLanes * kColsumWaves), 0, s, jobs);
    return hipGetLastError();
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
} // namespace

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    BwdLayout w;
    // the default forward's plan: one wave per slot at four waves per SIMD
    // (mamba130m_layer 22 parts, measured best among 16-64), parts of at most
    // 416 steps (long_seq 316 parts: 2 % faster than 128)
    w.p = default_fwd_plan(batch, L, dim);
    w.nck = (L + TT - 1) / TT;
    w.gpr = (dim + kLanes - 1) / kLanes;
    const size_t summ = (size_t)w.p.groups * (w.p.parts > 1 ? w.p.parts - 1 : 0) * (N + 1) *
                        kLanes * 4;
    const size_t slots = (size_t)batch * w.p.parts;
    size_t off = 0;
    const size_t entry = (size_t)w.p.groups * w.p.parts * N * kLanes * 4;
    // the forward's part summaries and entry states first, at the offsets
    // the default forward uses (summary_buffer, entry_buffer): a backward with
    // SELSCAN_FLAG_REUSE_FWD_STATE reads them where the forward left them
    w.fsumm = off; off = align256(off + summ);
    w.fentry = off; off = align256(off + entry);
    w.asumm = off; off = align256(off + summ);
    w.aentry = off; off = align256(off + entry);
    w.carry = off; off = align256(off + carry_scratch_bytes(w.p.groups, w.p.parts, N));
    w.ckpt = off; off = align256(off + (size_t)w.p.groups * w.nck * N * kLanes * 4);
    w.pB = off; off = align256(off + (size_t)w.gpr * batch * L * N * 4);
    w.pC = off; off = align256(off + (size_t)w.gpr * batch * L * N * 4);
    w.pA = off; off = align256(off + slots * dim * N * 4);
    w.pD = off; off = align256(off + slots * dim * 4);
    w.pbias = off; off = align256(off + slots * dim * 4);
    w.pW = off; off = align256(off + slots * dim * kMaxConv * 4);
    w.pWb = off; off = align256(off + slots * dim * 4);
    // the conv prologue's scan inputs and their gradients (fp32); every
    // variant shares one size query, so the buffer is always counted
    w.uconv = off; off = align256(off + (size_t)batch * L * dim * 4);
    w.total = off + 256;   // room to align the base
    return w;
}

} // namespace bwd

size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    return bwd::bwd_layout(batch, L, dim, N).total;
}

size_t bwd_checkpoint_offset(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    return bwd::bwd_layout(batch, L, dim, N).ckpt;
}

hipError_t launch_bwd_euler(const BwdArgs &a, const FwdExt &e, hipStream_t stream)
{
    return bwd::launch_bwd_var<0>(a, e, stream);
}

hipError_t launch_bwd(const BwdArgs &a, const FwdExt *e, hipStream_t stream)
{
    FwdExt none;
    none.flags = 0;
    none.conv_w = nullptr;
    none.conv_b = nullptr;
    none.conv_k = 0;
    const FwdExt &x = e ? *e : none;
    const bool zoh = (x.flags & kFwdFlagZohExact) != 0;
    if (x.conv_k > 0)
        return zoh ? launch_bwd_zoh_conv(a, x, stream) : launch_bwd_euler_conv(a, x, stream);
    if (zoh)
        return launch_bwd_zoh(a, x, stream);
    return (x.flags & kFwdFlagReverse) ? launch_bwd_euler_rev(a, x, stream)
                                       : launch_bwd_euler(a, x, stream);
}

} // namespace selscan
