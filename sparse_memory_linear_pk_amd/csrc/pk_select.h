// Per-row selection of product-key addressing (SDM blog post, caption of the
// figure "The SDM mechanism, end to end": two sub-keys, outer sum, top-k,
// softmax-weighted read), shared by the batched selection kernel (pk_topk) and
// the decode step's addressing (sdm_step).  One wave64 selects one row; every
// step is exact, with a general path behind each shortcut:
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
#pragma once

#include "sdm_internal.h"

namespace sdm {
namespace pksel {

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
__device__ inline uint32_t kth_largest(const uint32_t (&key)[J], int want, int rounds = 32)
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
__device__ inline int count_above(const uint32_t (&key)[J], uint32_t thr)
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
__device__ inline uint64_t half_sorted_topk(const float* __restrict__ s, int S, int k, int lane, uint64_t* buf)
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
__device__ inline void select_w(const uint32_t (&key)[M], const uint32_t (&slot)[M], int W, uint32_t thr, uint64_t* win)
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

// Restricted candidate pairs of k-long sorted lists for W winners: row i of the
// lists pairs with columns j < min(k, W / (i + 1)), listed row-major as
// (i << 8 | j).  Filled by all threads of a block.
__device__ inline void fill_pairs(uint16_t* pairs, int k, int W)
{
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        int off = 0;
        for (int r = 0; r < i; ++r)
            off += min(k, W / (r + 1));
        const int len = min(k, W / (i + 1));
        for (int j = 0; j < len; ++j)
            pairs[off + j] = (uint16_t)((i << 8) | j);
    }
}

inline int pair_count(int k, int W)
{
    int n = 0;
    for (int i = 0; i < k; ++i)
        n += W / (i + 1) < k ? W / (i + 1) : k;
    return n;
}

// Step 1 for one half by one wave: the half's sorted top k into val[lane] and
// sub[lane] (scores and sub-key indices, 64 entries; lanes past k hold padding).
template <int J>
__device__ inline void select_half(const float* s, int S, int k, int lane, uint64_t* buf, float* val, uint32_t* sub)
{
    const uint64_t x = half_sorted_topk<J>(s, S, k, lane, buf);
    val[lane] = key_value((uint32_t)(x >> 32));
    sub[lane] = ~(uint32_t)x;
}

// Step 2 by one wave, from both halves' sorted lists (val, sub: 2 x 64, in
// LDS and visible to the wave): idx_row, wt_row receive the W slots and
// weights, best first.  buf: 64 entries of the wave's LDS scratch.
template <int R>
__device__ inline void select_from_lists(int S, int k, int W, int n_pairs, const uint16_t* s_pairs, int lane,
                                         uint64_t* buf, const float (*val)[64], const uint32_t (*sub)[64],
                                         int32_t* idx_row, float* wt_row);

// The selection of one row by one wave: s holds the row's half scores (S of
// half 0, then S of half 1; global or LDS); buf, val, sub are the wave's LDS
// scratch (64 entries each, val and sub 2 x 64); idx_row, wt_row receive the W
// slots and weights, best first.
template <int J, int R>
__device__ inline void select_row(const float* s, int S, int k, int W, int n_pairs, const uint16_t* s_pairs,
                                  int lane, uint64_t* buf, float (*val)[64], uint32_t (*sub)[64],
                                  int32_t* idx_row, float* wt_row)
{
#pragma unroll
    for (int h = 0; h < 2; ++h)
        select_half<J>(s + h * S, S, k, lane, buf, val[h], sub[h]);
    wave_sync_lds();
    select_from_lists<R>(S, k, W, n_pairs, s_pairs, lane, buf, val, sub, idx_row, wt_row);
}

template <int R>
__device__ inline void select_from_lists(int S, int k, int W, int n_pairs, const uint16_t* s_pairs, int lane,
                                         uint64_t* buf, const float (*val)[64], const uint32_t (*sub)[64],
                                         int32_t* idx_row, float* wt_row)
{

    // restricted candidates
    uint32_t key[R], slot[R];
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int c = m * 64 + lane;
        key[m] = 0u;
        slot[m] = 0xFFFFFFFFu;
        if (c < n_pairs) {
            const int i = s_pairs[c] >> 8, j = s_pairs[c] & 0xFF;
            key[m] = ordered_key(val[0][i] + val[1][j]);
            slot[m] = sub[0][i] * (uint32_t)S + sub[1][j];
        }
    }
    const uint32_t thr_w = kth_largest<R>(key, W);
    // an excluded pair whose sum equals the W-th: the largest excluded sum of
    // list row i is at column W / (i + 1) (when that is < k)
    bool clash = false;
    if (lane < k) {
        const int j0 = W / (lane + 1);
        if (j0 < k)
            clash = ordered_key(val[0][lane] + val[1][j0]) == thr_w;
    }
    if (ballot(clash) == 0ull) {
        select_w<R>(key, slot, W, thr_w, buf);
    } else {
        // all k*k candidates, 64 at a time, recomputed for every round
        const int kk = k * k;
        auto cand = [&](int c, uint32_t& kc, uint32_t& sc) {
            kc = 0u;
            sc = 0xFFFFFFFFu;
            if (c < kk) {
                const int i = c / k, j = c - (c / k) * k;
                kc = ordered_key(val[0][i] + val[1][j]);
                sc = sub[0][i] * (uint32_t)S + sub[1][j];
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
                buf[p] = ((uint64_t)kc << 32) | (uint64_t)(~sc);
            placed += __popcll(sm);
        }
    }
    wave_sync_lds();

    // sort the W winners, descending by (sum, ~slot)
    const uint64_t x = sort64_desc(lane < W ? buf[lane] : 0ull, lane);
    // softmax in double over the sorted sums; lane 0 holds the largest
    const float sig = key_value((uint32_t)(x >> 32));
    const double mx = __shfl((double)sig, 0);
    double e = lane < W ? exp((double)sig - mx) : 0.0;
    double z = e;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        z += shfl_xor_f64(z, m);
    if (lane < W) {
        idx_row[lane] = (int32_t)(~(uint32_t)x);
        wt_row[lane] = (float)(e / z);
    }
}

} // namespace pksel
} // namespace sdm
