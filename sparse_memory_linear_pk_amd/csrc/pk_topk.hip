// pk_topk: the selection half of product-key addressing, for every row of a
// call: per half the k best sub-keys, the W best of their outer sums, softmax
// weights.  One wave64 per row runs pksel::select_row (pk_select.h has the
// algorithm and the argument for its exactness).  Given the queries and the
// sub-key tables (the forward's path), the scores that can reach a half's top k
// are first made exact (pksel::select_row_exact), so the slots and weights are
// those of exactly rounded scores; the stored scores only locate the
// candidates, and for bf16 inputs they are binary16.  Given scores alone (the
// stage seam), the float32 scores are taken as they are.
#include "pk_select.h"

#include <type_traits>

namespace sdm {
namespace {

using namespace pksel;

constexpr int kRowsPerBlock = 4; // one wave per row

// What the exact path reads: the queries [B, Ts, H, dk], the sub-key tables
// [H, 2, S, dh] and kAbsmaxParts partial maxima of |K| per table ([H, 2, parts]).
struct ExactIn {
    const void* q;
    const void* subkeys;
    const float* kmax;
    int dh;
};

// The outputs of one query set; blockIdx.y picks set 0 or 1 (q0 is ExactIn::q).
struct SetOut {
    const void* scores;
    int32_t* idx;
    float* wt;
    const void* q;
};

// J: sub-keys per lane per half (S <= 64*J); R: restricted candidates per lane;
// EX: 0 float32 scores as given, 1 exact from bf16 inputs (binary16 scores), 2
// exact from float32 inputs (float32 scores), 3 exact from bf16 inputs and the
// fused scoring's candidate records (in place of scores).
template <int J, int R, int EX>
__global__ __launch_bounds__(kRowsPerBlock * 64) void pk_topk_kernel(SetOut s0, SetOut s1, Rows rr, int S, int k,
                                                                   int W, int n_pairs, ExactIn ex)
{
    const SetOut& so = blockIdx.y ? s1 : s0;
    const void* __restrict__ scores_v = so.scores;
    int32_t* __restrict__ idx = so.idx;
    float* __restrict__ wt = so.wt;
    ex.q = so.q;
    __shared__ uint64_t s_buf[kRowsPerBlock][64];       // compaction scratch, then the winners
    __shared__ float s_val[kRowsPerBlock][2][64];        // sorted half lists: scores
    __shared__ uint32_t s_sub[kRowsPerBlock][2][64];     // and sub-key indices
    __shared__ uint16_t s_pairs[kPairsMax];              // restricted candidates
    // the rows' queries as doubles (exact path): dk per wave, dynamic, so that
    // the workgroup's LDS stays small enough for two of them per CU beside a
    // running scan
    extern __shared__ double s_qd[];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    fill_pairs(s_pairs, k, W);
    __syncthreads();

    const long j = (long)blockIdx.x * kRowsPerBlock + wave; // row of the chunk
    if (j >= rr.count())
        return; // whole wave leaves; no block-level barriers below
    const long per_seq = (long)rr.Tc * rr.H;
    const long row = ((j / per_seq) * rr.Ts + rr.t0) * rr.H + j % per_seq; // row (b, t, h) of the call
    if constexpr (EX == 0) {
        const float* scores = static_cast<const float*>(scores_v);
        select_row<J, R>(scores + row * 2 * (long)S, S, k, W, n_pairs, s_pairs, lane, s_buf[wave], s_val[wave],
                         s_sub[wave], idx + row * W, wt + row * W);
    } else {
        constexpr bool BF16 = EX == 1 || EX == 3;
        const int h = (int)(row % rr.H), dh = ex.dh;
        const size_t es = BF16 ? 2 : 4;
        double* qd = s_qd + (size_t)wave * 2 * dh;
        stage_query<BF16>(static_cast<const char*>(ex.q) + (size_t)row * 2 * dh * es, qd, 2 * dh, lane);
        const char* tab = static_cast<const char*>(ex.subkeys) + (size_t)h * 2 * S * dh * es;
        Refine r0{qd, tab, dh, 0.f}, r1{qd + dh, tab + (size_t)S * dh * es, dh, 0.f};
        r0.E = half_bound(r0, max_of_parts(ex.kmax + (h * 2 + 0) * kAbsmaxParts, kAbsmaxParts, lane), lane);
        r1.E = half_bound(r1, max_of_parts(ex.kmax + (h * 2 + 1) * kAbsmaxParts, kAbsmaxParts, lane), lane);
        using SC = std::conditional_t<BF16, uint16_t, float>;
        if constexpr (EX == 1) {
            r0.E = bound_f16(r0.E, dh);
            r1.E = bound_f16(r1.E, dh);
        }
        if constexpr (EX == 3) {
            const uint32_t* rec = static_cast<const uint32_t*>(scores_v);
            const long rows_all = (long)rr.B * rr.Ts * rr.H, rw = cand_record_dwords(S);
            select_row_cand<J, R, true>(rec + row * rw, rec + (rows_all + row) * rw, S, k, W, n_pairs, s_pairs, lane,
                                        s_buf[wave], s_val[wave], s_sub[wave], idx + row * W, wt + row * W, r0, r1);
        } else {
            const SC* scores = static_cast<const SC*>(scores_v);
            select_row_exact<J, R, BF16, false, SC>(scores + row * 2 * (long)S, S, k, W, n_pairs, s_pairs, lane,
                                                    s_buf[wave], s_val[wave], s_sub[wave], idx + row * W,
                                                    wt + row * W, r0, r1);
        }
    }
}

// Partial maxima of |K|: workgroup (table, part) covers the part-th of
// kAbsmaxParts equal slices of sub-key table (h, half) = blockIdx.x.
template <bool BF16>
__global__ __launch_bounds__(256) void subkey_absmax_kernel(const void* __restrict__ subkeys, float* __restrict__ kmax,
                                                            int S, int dh)
{
    __shared__ float s_red[4];
    const long n = (long)S * dh;
    const long base = (long)blockIdx.x * n;
    const long lo = n * blockIdx.y / kAbsmaxParts, hi = n * (blockIdx.y + 1) / kAbsmaxParts;
    float m = 0.f;
    for (long i = lo + threadIdx.x; i < hi; i += blockDim.x) {
        const float v = BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(subkeys)[base + i] << 16)
                             : static_cast<const float*>(subkeys)[base + i];
        m = fmaxf(m, fabsf(v));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0)
        s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        kmax[(long)blockIdx.x * kAbsmaxParts + blockIdx.y] =
            fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

template <int J, int EX>
hipError_t launch_j(const SetOut& s0, const SetOut& s1, int nsets, const Rows& r, int S, int k, int W, int n_pairs,
                    const ExactIn& ex, hipStream_t stream)
{
    dim3 grid((unsigned)((r.count() + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)nsets), block(kRowsPerBlock * 64);
    const size_t qd_bytes = EX ? (size_t)kRowsPerBlock * 2 * ex.dh * sizeof(double) : 0;
#define SDM_TOPK_R(Rv)                                                                                        \
    if (n_pairs <= 64 * Rv) {                                                                                 \
        hipLaunchKernelGGL((pk_topk_kernel<J, Rv, EX>), grid, block, qd_bytes, stream, s0, s1, r, S, k, W, n_pairs, ex); \
        return hipGetLastError();                                                                             \
    }
    SDM_TOPK_R(1)
    SDM_TOPK_R(2)
    SDM_TOPK_R(4)
    SDM_TOPK_R(8)
#undef SDM_TOPK_R
    return hipErrorInvalidValue;
}

template <int EX>
hipError_t launch_ex(const SetOut& s0, const SetOut& s1, int nsets, const Rows& r, int S, int k, int W, int n_pairs,
                     const ExactIn& ex, hipStream_t stream)
{
    if (S <= 64)
        return launch_j<1, EX>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    if (S <= 128)
        return launch_j<2, EX>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    if (S <= 256)
        return launch_j<4, EX>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    if (S <= 512)
        return launch_j<8, EX>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    if (S <= 1024)
        return launch_j<16, EX>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    return hipErrorInvalidValue;
}

// Both query sets' selection in one launch (nsets 2) or one set (nsets 1, s1 unused).
// cand: the sets' scores are the fused scoring's candidate records (bf16 inputs).
hipError_t launch_sets(const SetOut& s0, const SetOut& s1, int nsets, const Rows& r, int S, int k, int W,
                       const void* subkeys, const float* kmax, int dh, bool in_bf16, hipStream_t stream,
                       bool cand = false)
{
    if (r.count() <= 0)
        return hipSuccess;
    if (k < 1 || k > 64 || W < 1 || W > 64 || W > k * k || k > S)
        return hipErrorInvalidValue;
    const bool exact = s0.q != nullptr;
    if (exact && (!subkeys || !kmax || dh < 16 || dh % 16 || (nsets == 2 && !s1.q)))
        return hipErrorInvalidValue;
    const int n_pairs = pair_count(k, W);
    if (n_pairs > kPairsMax)
        return hipErrorInvalidValue;
    const ExactIn ex{s0.q, subkeys, kmax, dh};
    if (!exact)
        return launch_ex<0>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
    if (cand)
        return in_bf16 && pk_cand_path(S, dh, k, true) ? launch_ex<3>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream)
                                                       : hipErrorInvalidValue;
    return in_bf16 ? launch_ex<1>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream)
                   : launch_ex<2>(s0, s1, nsets, r, S, k, W, n_pairs, ex, stream);
}

} // namespace

hipError_t launch_subkey_absmax(const void* subkeys, float* kmax, int H, int S, int dh, bool in_bf16,
                                hipStream_t stream)
{
    const dim3 grid((unsigned)(2 * H), (unsigned)kAbsmaxParts);
    if (in_bf16)
        hipLaunchKernelGGL((subkey_absmax_kernel<true>), grid, dim3(256), 0, stream, subkeys, kmax, S, dh);
    else
        hipLaunchKernelGGL((subkey_absmax_kernel<false>), grid, dim3(256), 0, stream, subkeys, kmax, S, dh);
    return hipGetLastError();
}

hipError_t launch_pk_topk(const void* scores, int32_t* idx, float* wt, const Rows& r, int S, int k, int W,
                          const void* q, const void* subkeys, const float* kmax, int dh, bool in_bf16,
                          hipStream_t stream)
{
    const SetOut s0{scores, idx, wt, q};
    return launch_sets(s0, s0, 1, r, S, k, W, subkeys, kmax, dh, in_bf16, stream);
}

hipError_t launch_pk_topk_pair(const void* scores0, const void* scores1, int32_t* idx0, int32_t* idx1, float* wt0,
                               float* wt1, const Rows& r, int S, int k, int W, const void* q0, const void* q1,
                               const void* subkeys, const float* kmax, int dh, bool in_bf16, hipStream_t stream)
{
    if (!q0 || !q1)
        return hipErrorInvalidValue;
    const SetOut s0{scores0, idx0, wt0, q0}, s1{scores1, idx1, wt1, q1};
    return launch_sets(s0, s1, 2, r, S, k, W, subkeys, kmax, dh, in_bf16, stream);
}

hipError_t launch_pk_topk_cand(const void* rec0, const void* rec1, int32_t* idx0, int32_t* idx1, float* wt0,
                               float* wt1, int nsets, const Rows& r, int S, int k, int W, const void* q0,
                               const void* q1, const void* subkeys, const float* kmax, int dh, hipStream_t stream)
{
    if (!q0 || (nsets == 2 && !q1) || nsets < 1 || nsets > 2)
        return hipErrorInvalidValue;
    const SetOut s0{rec0, idx0, wt0, q0}, s1{nsets == 2 ? rec1 : rec0, nsets == 2 ? idx1 : idx0,
                                              nsets == 2 ? wt1 : wt0, nsets == 2 ? q1 : q0};
    return launch_sets(s0, s1, nsets, r, S, k, W, subkeys, kmax, dh, true, stream, true);
}

} // namespace sdm
