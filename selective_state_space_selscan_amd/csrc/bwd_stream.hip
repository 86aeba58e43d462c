// Backward of the selective scan: the reductions of the partials, the
// workspace layout, the dispatch over the variants and the instantiation for
// the Euler B_bar in the forward direction.  The kernels are in
// bwd_stream_impl.hpp.
#include "bwd_stream_impl.hpp"

namespace selscan {
namespace bwd {

// out[i] = sum_k in[k * P + i] for i < P, k < K: a block of four waves owns 64
// columns; wave w adds the rows k = w, w + 4, ... (eight loads in flight),
// then the four sums are added in wave order.
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const float *__restrict__ in,
                                                         float *__restrict__ out, int64_t P,
                                                         int64_t K)
{
    __shared__ float part[4][kLanes];
    const int lane = threadIdx.x & (kLanes - 1), wave = threadIdx.x >> 6;
    const int64_t i = (int64_t)blockIdx.x * kLanes + lane;
    float s = 0.0f;
    if (i < P) {
        int64_t k = wave;
        for (; k + 28 < K; k += 32) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = in[(k + 4 * j) * P + i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                s += v[j];
        }
        for (; k < K; k += 4)
            s += in[k * P + i];
    }
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && i < P)
        out[i] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

hipError_t launch_colsum(const float *in, float *out, int64_t P, int64_t K, hipStream_t s)
{
    if (!out || P <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(bwd_colsum_kernel, dim3((unsigned)((P + kLanes - 1) / kLanes)), dim3(256),
                       0, s, in, out, P, K);
    return hipGetLastError();
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
} // namespace

BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    BwdLayout w;
    w.p = make_stream_plan(batch, L, dim);
    w.nck = (L + TT - 1) / TT;
    w.gpr = (dim + kLanes - 1) / kLanes;
    const size_t summ = (size_t)w.p.groups * (w.p.parts > 1 ? w.p.parts - 1 : 0) * (N + 1) *
                        kLanes * 4;
    const size_t slots = (size_t)batch * w.p.parts;
    size_t off = 0;
    const size_t entry = (size_t)w.p.groups * w.p.parts * N * kLanes * 4;
    w.fsumm = off; off = align256(off + summ);
    w.asumm = off; off = align256(off + summ);
    w.fentry = off; off = align256(off + entry);
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
    w.xown = off; off = align256(off + (size_t)w.p.groups * w.p.parts * kHalo * kLanes * 4);
    w.xcarry = off; off = align256(off + (size_t)w.p.groups * w.p.parts * kHalo * kLanes * 4);
    w.total = off + 256;   // room to align the base
    return w;
}

} // namespace bwd

size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N)
{
    return bwd::bwd_layout(batch, L, dim, N).total;
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
