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
// One wave64 handles one row; every step is exact, with a general path behind
// each shortcut.
//
// Step 1, per half.  Lane L holds sub-keys j*64 + L.  The k-th largest of the
// 64 lane maxima is a lower bound of the half's k-th largest score (k distinct
// lanes reach it), so only the scores at or above it can survive.  A short
// radix select over one key per lane finds a bound no larger than that; the
// scores at or above it (about 45 of 480 at S = 480, k = 32) are compacted one
// per lane and sorted by a 64-lane bitonic network, which leaves the half's
// top k in order.  If more than 64 scores pass, an exact 32-round radix select
// over all of them finds the k survivors instead, and the same network sorts
// them.
//
// Step 2.  With both lists sorted, candidate (i, j) (i-th of half 0, j-th of
// half 1, from 0) is preceded by the (i+1)(j+1) - 1 pairs (i' <= i, j' <= j),
// whose sums are no smaller because float addition is monotone.  So the top W
// lie among the pairs with (i+1)(j+1) <= W (216 of 1024 at k = 32, W = 64),
// except where a sum outside that set equals the W-th sum exactly: rounding can
// equate the sums of different half scores, and then the slot order decides.
// One check per list row catches that case (the sums of an excluded pair are at
// most the W-th, and the largest excluded sum of row i is at column W/(i+1)),
// and the row then selects over all k*k candidates.  The W-th largest sum is
// found by a radix select on order-preserving keys; ties at it are taken in slot
// order by a second select.  The W winners are sorted by a 64-lane bitonic
// network on (sum, ~slot) and weighted by a softmax in double precision, so the
// float32 weights are the correctly rounded values of the exact softmax of the
// float32 sums, up to the rounding of exp.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row
constexpr int kPairsMax = 512;     // restricted candidates (at most ~300 for k, W <= 64)
constexpr int kBoundRounds = 16;   // radix rounds of the per-half lower bound

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ int rank_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Largest t such that at least `want` of the keys are >= t (the want-th largest
// key), resolved to the top `rounds` bits: with fewer than 32 rounds the result
// is a lower bound that still has `want` keys at or above it.  Items not in play
// carry key 0, below every float's key.
template <int J>
__device__ uint32_t kth_largest(const uint32_t (&key)[J], int want, int rounds = 32)
{
    uint32_t thr = 0;
    for (int bit = 31; bit > 31 - rounds; --bit) {
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

// Descending bitonic sort of one 64-bit value per lane across the wave.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t x, int lane)
{
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t y = shfl_xor64(x, stride);
            const bool take_max = ((lane & size) == 0) == ((lane & stride) == 0);
            x = take_max ? (x > y ? x : y) : (x < y ? x : y);
        }
    }
    return x;
}

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Top k of one half, sorted (score desc, index asc): lane r < k ends with the
// r-th survivor as (key << 32) | ~index.  buf: 64 entries of wave scratch.
template <int J>
__device__ uint64_t half_sorted_topk(const float* __restrict__ s, int S, int k, int lane, uint64_t* buf)
{
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int idx = j * 64 + lane;
        key[j] = idx < S ? ordered_key(s[idx]) : 0u;
    }
    uint32_t lane_max[1] = {0u};
#pragma unroll
    for (int j = 0; j < J; ++j)
        lane_max[0] = key[j] > lane_max[0] ? key[j] : lane_max[0];
    // with one key per lane the lane maxima are the scores: no bound is needed
    const uint32_t bound = J == 1 ? 0u : kth_largest<1>(lane_max, k, kBoundRounds);
    int passing = 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
        passing += __popcll(ballot(key[j] >= bound && key[j] != 0u));

    uint32_t thr = bound;
    int need = 64; // ties at thr to take (all of them on the compacting path)
    if (passing > 64) {
        // exact k-th largest, ties at it taken lowest index first
        thr = kth_largest<J>(key, k);
        need = k - count_above<J>(key, thr);
    }
    int tied = 0, placed = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const bool live = key[j] != 0u;
        const uint64_t eq = ballot(live && key[j] == thr);
        const bool take_tie = live && key[j] == thr && tied + rank_below(eq) < need;
        tied += __popcll(eq);
        const bool sel = live && (key[j] > thr || take_tie);
        const uint64_t sm = ballot(sel);
        const int p = placed + rank_below(sm);
        if (sel && p < 64)
            buf[p] = ((uint64_t)key[j] << 32) | (uint64_t)(~(uint32_t)(j * 64 + lane));
        placed += __popcll(sm);
    }
    wave_sync_lds();
    const uint64_t x = lane < placed ? buf[lane] : 0ull;
    wave_sync_lds();
    return sort64_desc(x, lane);
}

// The W best of M candidates per lane (key, slot), given thr, the W-th largest
// key: ties at thr taken in slot order; the winners go to win[0..W) unsorted.
template <int M>
__device__ void select_w(const uint32_t (&key)[M], const uint32_t (&slot)[M], int W, uint32_t thr, uint64_t* win)
{
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
        const bool sel = key[m] != 0u && (key[m] > thr || (key[m] == thr && (n_eq == need || ~slot[m] >= slot_thr)));
        const uint64_t sm = ballot(sel);
        const int p = placed + rank_below(sm);
        if (sel && p < 64)
            win[p] = ((uint64_t)key[m] << 32) | (uint64_t)(~slot[m]);
        placed += __popcll(sm);
    }
}

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
    __shared__ uint16_t s_pairs[kPairsMax];              // restricted candidates (i << 8 | j), row-major

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // row i of the sorted lists pairs with columns j < min(k, W / (i + 1))
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        int off = 0;
        for (int r = 0; r < i; ++r)
            off += min(k, W / (r + 1));
        const int len = min(k, W / (i + 1));
        for (int j = 0; j < len; ++j)
            s_pairs[off + j] = (uint16_t)((i << 8) | j);
    }
    __syncthreads();

    const long j = (long)blockIdx.x * kRowsPerBlock + wave; // row of the chunk
    if (j >= rr.count())
        return; // whole wave leaves; no block-level barriers below
    const long per_seq = (long)rr.Tc * rr.H;
    const long row = ((j / per_seq) * rr.Ts + rr.t0) * rr.H + j % per_seq; // row (b, t, h) of the call

    const float* s = scores + row * 2 * (long)S;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint64_t x = half_sorted_topk<J>(s + h * S, S, k, lane, s_buf[wave]);
        s_val[wave][h][lane] = key_value((uint32_t)(x >> 32));
        s_sub[wave][h][lane] = ~(uint32_t)x;
    }
    wave_sync_lds();

    // restricted candidates
    uint32_t key[R], slot[R];
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int c = m * 64 + lane;
        key[m] = 0u;
        slot[m] = 0xFFFFFFFFu;
        if (c < n_pairs) {
            const int i = s_pairs[c] >> 8, j = s_pairs[c] & 0xFF;
            key[m] = ordered_key(s_val[wave][0][i] + s_val[wave][1][j]);
            slot[m] = s_sub[wave][0][i] * (uint32_t)S + s_sub[wave][1][j];
        }
    }
    const uint32_t thr_w = kth_largest<R>(key, W);
    // an excluded pair whose sum equals the W-th: the largest excluded sum of
    // list row i is at column W / (i + 1) (when that is < k)
    bool clash = false;
    if (lane < k) {
        const int j0 = W / (lane + 1);
        if (j0 < k)
            clash = ordered_key(s_val[wave][0][lane] + s_val[wave][1][j0]) == thr_w;
    }
    if (ballot(clash) == 0ull) {
        select_w<R>(key, slot, W, thr_w, s_buf[wave]);
    } else {
        // all k*k candidates, 64 at a time, recomputed for every round
        const int kk = k * k;
        auto cand = [&](int c, uint32_t& kc, uint32_t& sc) {
            kc = 0u;
            sc = 0xFFFFFFFFu;
            if (c < kk) {
                const int i = c / k, j = c - (c / k) * k;
                kc = ordered_key(s_val[wave][0][i] + s_val[wave][1][j]);
                sc = s_sub[wave][0][i] * (uint32_t)S + s_sub[wave][1][j];
            }
        };
        const int nm = (kk + 63) / 64;
        uint32_t thr = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cnd = thr | (1u << bit);
            int cnt = 0;
            for (int m = 0; m < nm; ++m) {
                uint32_t kc, sc;
                cand(m * 64 + lane, kc, sc);
                cnt += __popcll(ballot(kc >= cnd));
            }
            if (cnt >= W)
                thr = cnd;
        }
        int above = 0, n_eq = 0;
        for (int m = 0; m < nm; ++m) {
            uint32_t kc, sc;
            cand(m * 64 + lane, kc, sc);
            above += __popcll(ballot(kc > thr));
            n_eq += __popcll(ballot(kc == thr));
        }
        const int need = W - above;
        uint32_t slot_thr = 0u;
        if (n_eq > need) {
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cnd = slot_thr | (1u << bit);
                int cnt = 0;
                for (int m = 0; m < nm; ++m) {
                    uint32_t kc, sc;
                    cand(m * 64 + lane, kc, sc);
                    cnt += __popcll(ballot(kc == thr && ~sc >= cnd));
                }
                if (cnt >= need)
                    slot_thr = cnd;
            }
        }
        int placed = 0;
        for (int m = 0; m < nm; ++m) {
            uint32_t kc, sc;
            cand(m * 64 + lane, kc, sc);
            const bool sel = kc != 0u && (kc > thr || (kc == thr && (n_eq == need || ~sc >= slot_thr)));
            const uint64_t sm = ballot(sel);
            const int p = placed + rank_below(sm);
            if (sel && p < 64)
                s_buf[wave][p] = ((uint64_t)kc << 32) | (uint64_t)(~sc);
            placed += __popcll(sm);
        }
    }
    wave_sync_lds();

    // sort the W winners, descending by (sum, ~slot)
    const uint64_t x = sort64_desc(lane < W ? s_buf[wave][lane] : 0ull, lane);
    // softmax in double over the sorted sums; lane 0 holds the largest
    const float sig = key_value((uint32_t)(x >> 32));
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
    int n_pairs = 0;
    for (int i = 0; i < k; ++i)
        n_pairs += W / (i + 1) < k ? W / (i + 1) : k;
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
