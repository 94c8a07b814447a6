// pk_topk: the selection half of product-key addressing.
//
// For one row (one query), from its two half-score vectors:
//   1. per half, keep the k sub-keys with the largest scores;
//   2. every pair (a, b) of survivors is a candidate slot n = a*S + b, scored by
//      the float32 sum of its two half scores (the outer sum);
//   3. keep the W best candidates and weight them by a softmax of their sums.
// Orders are by score descending and then by index ascending, so equal scores
// go to the lower sub-key or slot index.  (SDM blog post, caption of the figure
// "The SDM mechanism, end to end": two sub-keys, outer sum, top-k, softmax-
// weighted read; the tie order and the slot numbering are this library's
// reading, shared with its tests.)
//
// One wave64 handles one row.  A k-th largest value is found exactly by a
// radix select on order-preserving integer keys: 32 rounds, each a wave-wide
// count of keys at or above a candidate prefix (one v_cmp + popcount per item).
// Ties at the threshold are taken in index order with ballots.  The W winners
// are sorted with a 64-lane bitonic network on (key, ~slot) and weighted with an
// exact-in-double softmax, so the float32 weights match a double reference.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kRowsPerBlock = 4; // one wave per row

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ int rank_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Largest t such that at least `want` of the keys are >= t (the want-th largest key).
// Items not in play carry key 0, below every float's key.
template <int J>
__device__ uint32_t kth_largest(const uint32_t (&key)[J], int want)
{
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < J; ++j)
            cnt += __popcll(ballot(key[j] >= cand));
        if (cnt >= want)
            thr = cand;
    }
    return thr;
}

template <int J>
__device__ int count_above(const uint32_t (&key)[J], uint32_t thr)
{
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
        cnt += __popcll(ballot(key[j] > thr));
    return cnt;
}

// Top-k of one half: writes the k survivors (index, score) to lds_idx/lds_val
// in ascending index order.  Item j of lane L is sub-key j*64 + L.
template <int J>
__device__ void half_topk(const float* __restrict__ s, int S, int k, int lane, int32_t* lds_idx, float* lds_val)
{
    float val[J];
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int idx = j * 64 + lane;
        val[j] = idx < S ? s[idx] : 0.f;
        key[j] = idx < S ? ordered_key(val[j]) : 0u;
    }
    const uint32_t thr = kth_largest<J>(key, k);
    const int need = k - count_above<J>(key, thr); // ties at thr to take, lowest index first
    int tied = 0, placed = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const uint64_t eq = ballot(key[j] == thr);
        const bool take_tie = key[j] == thr && tied + rank_below(eq) < need;
        tied += __popcll(eq);
        const bool sel = key[j] > thr || take_tie;
        const uint64_t sm = ballot(sel);
        const int p = placed + rank_below(sm);
        if (sel && p < 64) {
            lds_idx[p] = j * 64 + lane;
            lds_val[p] = val[j];
        }
        placed += __popcll(sm);
    }
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m)
{
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m)
{
    return __longlong_as_double((long long)shfl_xor64((uint64_t)__double_as_longlong(x), m));
}

// J: items per lane for one half (S <= 64*J); M: candidates per lane (k*k <= 64*M)
template <int J, int M>
__global__ __launch_bounds__(kRowsPerBlock * 64) void pk_topk_kernel(const float* __restrict__ scores,
                                                                   int32_t* __restrict__ idx,
                                                                   float* __restrict__ wt, long rows, int S,
                                                                   int k, int W)
{
    __shared__ int32_t s_idx[kRowsPerBlock][2][64];
    __shared__ float s_val[kRowsPerBlock][2][64];
    __shared__ uint64_t s_win[kRowsPerBlock][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long row = (long)blockIdx.x * kRowsPerBlock + wave;
    if (row >= rows)
        return; // whole wave leaves; no block-level barriers below

    const float* s = scores + row * 2 * (long)S;
    half_topk<J>(s, S, k, lane, s_idx[wave][0], s_val[wave][0]);
    half_topk<J>(s + S, S, k, lane, s_idx[wave][1], s_val[wave][1]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // candidates: c = m*64 + lane -> (i, j) = (c / k, c % k)
    const int kk = k * k;
    uint32_t key[M];
    uint32_t slot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int c = m * 64 + lane;
        if (c < kk) {
            const int i = c / k, j = c - (c / k) * k;
            const float sum = s_val[wave][0][i] + s_val[wave][1][j];
            key[m] = ordered_key(sum);
            slot[m] = (uint32_t)(s_idx[wave][0][i] * S + s_idx[wave][1][j]);
        } else {
            key[m] = 0u;
            slot[m] = 0xFFFFFFFFu;
        }
    }
    const uint32_t thr = kth_largest<M>(key, W);
    const int need = W - count_above<M>(key, thr);
    int n_eq = 0;
#pragma unroll
    for (int m = 0; m < M; ++m)
        n_eq += __popcll(ballot(key[m] == thr));
    // among candidates tied at thr take the `need` lowest slots: the need-th largest of ~slot
    uint32_t slot_thr = 0u;
    if (n_eq > need) {
        uint32_t inv[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            inv[m] = key[m] == thr ? ~slot[m] : 0u;
        slot_thr = kth_largest<M>(inv, need);
    }
    int placed = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const bool sel = key[m] > thr || (key[m] == thr && (n_eq == need || ~slot[m] >= slot_thr));
        const uint64_t sm = ballot(sel);
        const int p = placed + rank_below(sm);
        if (sel && p < 64)
            s_win[wave][p] = ((uint64_t)key[m] << 32) | (uint64_t)(~slot[m]);
        placed += __popcll(sm);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // bitonic sort of the W winners across the wave, descending by (key, ~slot)
    uint64_t x = lane < W ? s_win[wave][lane] : 0ull;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t y = shfl_xor64(x, stride);
            const bool take_max = ((lane & size) == 0) == ((lane & stride) == 0);
            x = take_max ? (x > y ? x : y) : (x < y ? x : y);
        }
    }
    // softmax in double over the sorted sums; lane 0 holds the largest
    const uint32_t kx = (uint32_t)(x >> 32);
    const float sig = __uint_as_float((kx & 0x80000000u) ? (kx & 0x7FFFFFFFu) : ~kx);
    const double mx = __shfl((double)sig, 0);
    double e = lane < W ? exp((double)sig - mx) : 0.0;
    double z = e;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        z += shfl_xor_f64(z, m);
    if (lane < W) {
        idx[row * W + lane] = (int32_t)(~(uint32_t)x);
        wt[row * W + lane] = (float)(e / z);
    }
}

template <int J>
hipError_t launch_j(const float* scores, int32_t* idx, float* wt, long rows, int S, int k, int W,
                    hipStream_t stream)
{
    const int kk = k * k;
    dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
#define SDM_TOPK_M(Mv)                                                                                       \
    if (kk <= 64 * Mv) {                                                                                     \
        hipLaunchKernelGGL((pk_topk_kernel<J, Mv>), grid, block, 0, stream, scores, idx, wt, rows, S, k, W); \
        return hipGetLastError();                                                                            \
    }
    SDM_TOPK_M(1)
    SDM_TOPK_M(2)
    SDM_TOPK_M(4)
    SDM_TOPK_M(8)
    SDM_TOPK_M(16)
    SDM_TOPK_M(32)
    SDM_TOPK_M(64)
#undef SDM_TOPK_M
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_pk_topk(const float* scores, int32_t* idx, float* wt, long rows, int S, int k, int W,
                          hipStream_t stream)
{
    if (rows <= 0)
        return hipSuccess;
    if (S <= 64)
        return launch_j<1>(scores, idx, wt, rows, S, k, W, stream);
    if (S <= 128)
        return launch_j<2>(scores, idx, wt, rows, S, k, W, stream);
    if (S <= 256)
        return launch_j<4>(scores, idx, wt, rows, S, k, W, stream);
    if (S <= 512)
        return launch_j<8>(scores, idx, wt, rows, S, k, W, stream);
    if (S <= 1024)
        return launch_j<16>(scores, idx, wt, rows, S, k, W, stream);
    return hipErrorInvalidValue;
}

} // namespace sdm
