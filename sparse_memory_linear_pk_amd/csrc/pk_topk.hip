// pk_topk: the selection half of product-key addressing, for every row of a
// call: per half the k best sub-keys, the W best of their outer sums, softmax
// weights.  One wave64 per row runs pksel::select_row (pk_select.h has the
// algorithm and the argument for its exactness).
#include "pk_select.h"

namespace sdm {
namespace {

using namespace pksel;

constexpr int kRowsPerBlock = 4; // one wave per row

// J: sub-keys per lane per half (S <= 64*J); R: restricted candidates per lane.
template <int J, int R>
__global__ __launch_bounds__(kRowsPerBlock * 64) void pk_topk_kernel(const float* __restrict__ scores,
                                                                   int32_t* __restrict__ idx,
                                                                   float* __restrict__ wt, Rows rr, int S,
                                                                   int k, int W, int n_pairs)
{
    __shared__ uint64_t s_buf[kRowsPerBlock][64];       // compaction scratch, then the winners
    __shared__ float s_val[kRowsPerBlock][2][64];        // sorted half lists: scores
    __shared__ uint32_t s_sub[kRowsPerBlock][2][64];     // and sub-key indices
    __shared__ uint16_t s_pairs[kPairsMax];              // restricted candidates

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    fill_pairs(s_pairs, k, W);
    __syncthreads();

    const long j = (long)blockIdx.x * kRowsPerBlock + wave; // row of the chunk
    if (j >= rr.count())
        return; // whole wave leaves; no block-level barriers below
    const long per_seq = (long)rr.Tc * rr.H;
    const long row = ((j / per_seq) * rr.Ts + rr.t0) * rr.H + j % per_seq; // row (b, t, h) of the call
    select_row<J, R>(scores + row * 2 * (long)S, S, k, W, n_pairs, s_pairs, lane, s_buf[wave], s_val[wave],
                     s_sub[wave], idx + row * W, wt + row * W);
}

template <int J>
hipError_t launch_j(const float* scores, int32_t* idx, float* wt, const Rows& r, int S, int k, int W, int n_pairs,
                    hipStream_t stream)
{
    dim3 grid((unsigned)((r.count() + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
#define SDM_TOPK_R(Rv)                                                                                       \
    if (n_pairs <= 64 * Rv) {                                                                                \
        hipLaunchKernelGGL((pk_topk_kernel<J, Rv>), grid, block, 0, stream, scores, idx, wt, r, S, k, W,    \
                           n_pairs);                                                                         \
        return hipGetLastError();                                                                            \
    }
    SDM_TOPK_R(1)
    SDM_TOPK_R(2)
    SDM_TOPK_R(4)
    SDM_TOPK_R(8)
#undef SDM_TOPK_R
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_pk_topk(const float* scores, int32_t* idx, float* wt, const Rows& r, int S, int k, int W,
                          hipStream_t stream)
{
    if (r.count() <= 0)
        return hipSuccess;
    if (k < 1 || k > 64 || W < 1 || W > 64 || W > k * k || k > S)
        return hipErrorInvalidValue;
    const int n_pairs = pair_count(k, W);
    if (n_pairs > kPairsMax)
        return hipErrorInvalidValue;
    if (S <= 64)
        return launch_j<1>(scores, idx, wt, r, S, k, W, n_pairs, stream);
    if (S <= 128)
        return launch_j<2>(scores, idx, wt, r, S, k, W, n_pairs, stream);
    if (S <= 256)
        return launch_j<4>(scores, idx, wt, r, S, k, W, n_pairs, stream);
    if (S <= 512)
        return launch_j<8>(scores, idx, wt, r, S, k, W, n_pairs, stream);
    if (S <= 1024)
        return launch_j<16>(scores, idx, wt, r, S, k, W, n_pairs, stream);
    return hipErrorInvalidValue;
}

} // namespace sdm
