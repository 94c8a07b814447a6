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
//
// Exact scores (the forward's path, select_half with a Refine).  The scores from
// the matrix cores are float32 sums; they only locate the candidates.  Every
// score that can reach a half's top k is recomputed exactly: the dh products
// (exact in double for bf16 and float32 inputs) summed in double in index
// order and rounded once to float32, which is the definition the oracle
// computes, operation for operation.  Which scores can reach the top k: if E
// bounds |approximate - exact| for every score of the half, and beta is the
// lower bound of step 1 (k scores have approximate values >= beta), the k-th
// largest exact score is at least beta - E, so every member of the exact top k
// has an approximate score >= beta - 2E, and every score below that is
// strictly below the k-th exact one.  Those candidates (about the same 45 at
// S = 480, k = 32) are made exact and sorted; more than 64 of them (heavy ties)
// makes every score of the half exact and selects over all of them.  E is
// 2 (dh + 2) 2^-24 sum_c |q_c| max |K|: the recursive-summation bound of a
// dh-term float32 dot product in any order, plus the rounding of the exact one,
// doubled.
#pragma once

#include "sdm_internal.h"

namespace sdm {
namespace pksel {

constexpr int kPairsMax = 512;     // restricted candidates (at most ~300 for k, W <= 64)
constexpr int kBoundRounds = 16;   // radix rounds of the per-half lower bound

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// A stored score as float: float32 as it is, or binary16 bits (the forward's
// score buffer for bf16 inputs), which float holds exactly.
__device__ __forceinline__ float score_at(const float* s, int i) { return s[i]; }
__device__ __forceinline__ float score_at(const uint16_t* s, int i)
{
    return (float)__builtin_bit_cast(_Float16, s[i]);
}

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
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[J], int want, int rounds = 32)
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
__device__ __forceinline__ int count_above(const uint32_t (&key)[J], uint32_t thr)
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

// A counting form of the sort, for a wave that has its SIMD to itself (the
// decode step): every lane compares its key with all 64 from LDS.  That is more
// instructions than the bitonic network, but they are independent of one
// another, where the network is a chain of 21 dependent exchanges that a lone
// wave cannot hide.  The result is the same.
// sort64_desc for keys that are distinct where nonzero (zeros are padding and
// end up last): a key's place is the number of keys above it.  buf: 64
// entries of wave scratch.
__device__ __forceinline__ uint64_t sort64_desc_count(uint64_t x, int lane, uint64_t* buf)
{
    buf[lane] = x;
    wave_sync_lds();
    int gt = 0;
#pragma unroll
    for (int c = 0; c < 64; c += 2) {
        const uint4 y = *reinterpret_cast<const uint4*>(buf + c);
        gt += (int)((((uint64_t)y.y << 32) | y.x) > x) + (int)((((uint64_t)y.w << 32) | y.z) > x);
    }
    const int n = __popcll(ballot(x != 0ull));
    wave_sync_lds();
    if (x != 0ull)
        buf[gt] = x;
    wave_sync_lds();
    const uint64_t r = lane < n ? buf[lane] : 0ull;
    wave_sync_lds();
    return r;
}

// Exact score of a query half against one sub-key row: products summed in
// double in index order, rounded once to float32.  qd: the query half as
// doubles in LDS (stage_query).  The row streams through a ring of three
// 16-byte pieces, each loaded two pieces before its products, which keeps the
// registers of the selection (and so the waves per SIMD that hide the latency
// of its dependent steps) close to those of the selection from given scores.
template <bool BF16>
__device__ __forceinline__ float exact_score(const double* __restrict__ qd, const void* krow, int dh)
{
    constexpr int EPP = BF16 ? 8 : 4; // elements per 16-byte piece
    const uint4* kp = static_cast<const uint4*>(krow);
    const int np = dh / EPP;          // at least 2 (dh >= 16)
    double acc = 0.0;
    uint4 p0 = kp[0], p1 = kp[1];
    for (int c = 0; c < np; ++c) {
        const uint4 b = p0;
        p0 = p1;
        p1 = kp[min(c + 2, np - 1)]; // past the row: its last piece again, not used
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (BF16) {
                acc = fma(qd[c * EPP + 2 * w], (double)bf16_lo(bw[w]), acc);
                acc = fma(qd[c * EPP + 2 * w + 1], (double)bf16_hi(bw[w]), acc);
            } else {
                acc = fma(qd[c * EPP + w], (double)__uint_as_float(bw[w]), acc);
            }
        }
    }
    return __double2float_rn(acc);
}

// A query of dk elements (bf16 or float32) converted by one wave to doubles in
// its LDS buffer qd (dk doubles).
template <bool BF16>
__device__ __forceinline__ void stage_query(const void* q, double* qd, int dk, int lane)
{
    for (int c = lane; c < dk; c += 64)
        qd[c] = BF16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(q)[c] << 16)
                     : (double)static_cast<const float*>(q)[c];
    wave_sync_lds();
}

// What the exact path of one half needs: the row's query half as doubles (in
// LDS), the half's sub-key table [S, dh] and E, the bound on |approximate -
// exact| of its scores.
struct Refine {
    const double* qd;
    const void* table;
    int dh;
    float E;
};

// The largest of n partial maxima (n <= 64), on every lane.
__device__ __forceinline__ float max_of_parts(const float* part, int n, int lane)
{
    float m = lane < n ? part[lane] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    return m;
}

// sum_c |q_c| over a query half of dh doubles, on every lane.
__device__ __forceinline__ double abs_sum(const double* qd, int dh, int lane)
{
    double a = 0.0;
    for (int c = lane; c < dh; c += 64)
        a += fabs(qd[c]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        a += shfl_xor_f64(a, m);
    return a;
}

// E for a query half: 2 (dh + 2) 2^-24 sum_c |q_c| kmax, kmax = max |K| over
// the half's table.
__device__ __forceinline__ float bound_from(double abs_q, int dh, float kmax)
{
    return (float)(2.0 * (double)(dh + 2) * 0x1p-24 * abs_q * (double)kmax);
}

__device__ __forceinline__ float half_bound(const Refine& r, float kmax, int lane)
{
    return bound_from(abs_sum(r.qd, r.dh, lane), r.dh, kmax);
}

// The largest float32 no larger than x.
__device__ __forceinline__ float float_down(double x)
{
    float f = __double2float_rn(x);
    if ((double)f > x) { // one float step down
        const float z = f;
        uint32_t u = __float_as_uint(f);
        u = z > 0.f ? u - 1u : (z < 0.f ? u + 1u : 0x80000001u);
        f = __uint_as_float(u);
    }
    return f;
}

// Binary16 scores.  The float32 score s32 of a sub-key is stored rounded to
// binary16, h = f16(s32), so |h - s| <= E0 + r |h| for the exact score s, with
// E0 = E + 2^-24 (E bounds |s32 - s|; 2^-24 covers binary16's subnormal step)
// and r = 2^-10 (binary16 rounds to 11 significant bits, and |s32| <= |h| /
// (1 - 2^-11)).  If k stored scores are >= beta, each has s >= f(h) - E0 >=
// f(beta) - E0 with f(x) = x - r |x| (increasing), so the k-th largest exact
// score is at least L = f(beta) - E0.  A member of the exact top k then has
// g(h) >= s - E0 >= L - E0 with g(x) = x + r |x| (increasing), i.e. h >=
// g^-1(L - E0): every stored score below that is out.
__device__ __forceinline__ double threshold_f16(float beta, float E)
{
    const double r = 0x1p-10, e0 = (double)E + 0x1p-24;
    const double b = beta;
    const double y = (b - r * fabs(b)) - 2.0 * e0;
    return y >= 0.0 ? y / (1.0 + r) : y / (1.0 - r);
}

// E for the binary16 path: a half whose scores may leave binary16's range
// (|s| could reach 65504) gets an infinite bound, which makes every score of
// the half a candidate and every score exact.
__device__ __forceinline__ float bound_f16(float E, int dh)
{
    const double a = (double)E / (2.0 * (double)(dh + 2) * 0x1p-24); // sum_c |q_c| max |K|
    return a < 32768.0 ? E : __builtin_inff();
}

template <int J, bool BF16>
__device__ __forceinline__ uint64_t half_all_exact(int S, int k, int lane, uint64_t* buf, Refine ref);

// Top k of one half, sorted (score desc, index asc): lane r < k ends with the
// r-th survivor as (key << 32) | ~index.  buf: 64 entries of wave scratch.
// With ref, the scores that can reach the top k are made exact first (see the
// header): the survivors and their keys are those of the exact scores.
// LAT: the counting sort (a wave alone on its SIMD).
// SC: float (float32 scores) or uint16_t (binary16 scores; see threshold_f16).
template <int J, bool BF16, bool LAT = false, class SC = float>
__device__ __forceinline__ uint64_t half_sorted_topk_exact(const SC* __restrict__ s, int S, int k, int lane,
                                                           uint64_t* buf, Refine ref)
{
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int idx = j * 64 + lane;
        key[j] = idx < S ? ordered_key(score_at(s, idx)) : 0u;
    }
    uint32_t lane_max[1] = {0u};
#pragma unroll
    for (int j = 0; j < J; ++j)
        lane_max[0] = key[j] > lane_max[0] ? key[j] : lane_max[0];
    // with one key per lane every score is a candidate
    uint32_t thr = 0u;
    if (J > 1) {
        const uint32_t bound = kth_largest<1>(lane_max, k, kBoundRounds);
        const float beta = key_value(bound);
        const double lo = sizeof(SC) == 2 ? threshold_f16(beta, ref.E) : (double)beta - 2.0 * (double)ref.E;
        // a NaN bound (NaN scores) takes every score
        thr = lo == lo ? ordered_key(float_down(lo)) : 0u;
    }
    int passing = 0;
#pragma unroll
    for (int j = 0; j < J; ++j)
        passing += __popcll(ballot(key[j] != 0u && key[j] >= thr));
    const char* table = static_cast<const char*>(ref.table);
    const size_t row_bytes = (size_t)ref.dh * (BF16 ? 2 : 4);
    if (passing <= 64) {
        int placed = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool sel = key[j] != 0u && key[j] >= thr;
            const uint64_t sm = ballot(sel);
            if (sel)
                buf[placed + rank_below(sm)] = (uint64_t)(j * 64 + lane);
            placed += __popcll(sm);
        }
        wave_sync_lds();
        uint64_t x = 0ull;
        if (lane < placed) {
            const uint32_t sk = (uint32_t)buf[lane];
            const void* krow = table + sk * row_bytes;
            // rows of 256 bytes (bf16 halves of 128, float32 halves of 64) with every load up front
            const float e = exact_score<BF16>(ref.qd, krow, ref.dh);
            x = ((uint64_t)ordered_key(e) << 32) | (uint64_t)(~sk);
        }
        wave_sync_lds();
        return LAT ? sort64_desc_count(x, lane, buf) : sort64_desc(x, lane);
    }
    // heavy ties: every score of the half exact, the k-th largest by a full radix select
    return half_all_exact<J, BF16>(S, k, lane, buf, ref);
}

// Top k of one half with every score made exact, the k-th largest by a full
// radix select, ties at it taken lowest index first; sorted as
// half_sorted_topk_exact's result.
template <int J, bool BF16>
__device__ __forceinline__ uint64_t half_all_exact(int S, int k, int lane, uint64_t* buf, Refine ref)
{
    const char* table = static_cast<const char*>(ref.table);
    const size_t row_bytes = (size_t)ref.dh * (BF16 ? 2 : 4);
    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int idx = j * 64 + lane;
        key[j] = idx < S ? ordered_key(exact_score<BF16>(ref.qd, table + idx * row_bytes, ref.dh)) : 0u;
    }
    const uint32_t thr = kth_largest<J>(key, k);
    const int need = k - count_above<J>(key, thr);
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

// Sub-key of bit p of candidate word c (the fused scoring's record layout):
// bits 0-15 from lane group 0, 16-31 from group 1, each group's first score in
// its highest bit; within the 32-wide tile, score v of group g is sub-key
// 8 (v / 4) + 4 g + (v % 4).
__device__ __forceinline__ uint32_t cand_subkey(int c, int p)
{
    const int g = p >> 4, v = 15 - (p & 15);
    return (uint32_t)(c * 32 + 8 * (v >> 2) + 4 * g + (v & 3));
}

// Top k of one half from a candidate record: the sub-keys whose float32 score
// reached the record's threshold tau are made exact.  If at least k of them have
// exact scores >= tau + E, the k-th largest exact score is at least tau + E, so
// every sub-key that ties or beats it has a float32 score >= tau (E bounds the
// difference) and is a candidate: the sorted candidates then start with the
// exact top k.  Otherwise, or with more than 64 candidates, or an E too large to
// rule out float32 overflow in the scores, every score of the half is made
// exact.  rec: the record (S / 32 words, then tau); sorted as
// half_sorted_topk_exact's result.
template <int J, bool BF16>
__device__ __forceinline__ uint64_t half_sorted_topk_cand(const uint32_t* __restrict__ rec, int S, int k, int lane,
                                                          uint64_t* buf, Refine ref)
{
    const int nw = S / 32;
    uint32_t bits = lane < nw ? rec[lane] : 0u;
    const float tau = __uint_as_float(rec[nw]);
    const int cnt = __popc(bits);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        incl += lane >= o ? t : 0;
    }
    const int total = __shfl(incl, 63);
    if (total >= k && total <= 64 && ref.E < 1e30f) {
        int pos = incl - cnt;
        while (bits) {
            const int p = __ffs(bits) - 1;
            bits &= bits - 1u;
            buf[pos++] = (uint64_t)cand_subkey(lane, p);
        }
        wave_sync_lds();
        const char* table = static_cast<const char*>(ref.table);
        const size_t row_bytes = (size_t)ref.dh * (BF16 ? 2 : 4);
        uint64_t x = 0ull;
        float e = 0.f;
        if (lane < total) {
            const uint32_t sk = (uint32_t)buf[lane];
            e = exact_score<BF16>(ref.qd, table + sk * row_bytes, ref.dh);
            x = ((uint64_t)ordered_key(e) << 32) | (uint64_t)(~sk);
        }
        // tau + E in double, nudged up past its rounding (and past subnormal flushes)
        double lim = (double)tau + (double)ref.E;
        lim += fabs(lim) * 0x1p-50 + 0x1p-110;
        const bool ok = __popcll(ballot(lane < total && (double)e >= lim)) >= k;
        wave_sync_lds();
        if (ok)
            return sort64_desc(x, lane);
    }
    return half_all_exact<J, BF16>(S, k, lane, buf, ref);
}


// Top k of one half, sorted (score desc, index asc): lane r < k ends with the
// r-th survivor as (key << 32) | ~index.  buf: 64 entries of wave scratch.
template <int J>
__device__ __forceinline__ uint64_t half_sorted_topk(const float* __restrict__ s, int S, int k, int lane, uint64_t* buf)
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
__device__ __forceinline__ void select_w(const uint32_t (&key)[M], const uint32_t (&slot)[M], int W, uint32_t thr, uint64_t* win)
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
// (i << 8 | j).  Written by the block's last wave (lane i: row i, from where
// a prefix sum over the lanes' row lengths puts it); visible to the block after
// a barrier.
__device__ inline void fill_pairs(uint16_t* pairs, int k, int W)
{
    const int i = (int)threadIdx.x - ((int)blockDim.x - 64);
    if (i >= 0) {
        const int len = i < k ? min(k, W / (i + 1)) : 0;
        int end = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(end, o);
            end += i >= o ? t : 0;
        }
        for (int j = 0; j < len; ++j)
            pairs[end - len + j] = (uint16_t)((i << 8) | j);
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
__device__ __forceinline__ void select_half(const float* s, int S, int k, int lane, uint64_t* buf, float* val, uint32_t* sub)
{
    const uint64_t x = half_sorted_topk<J>(s, S, k, lane, buf);
    val[lane] = key_value((uint32_t)(x >> 32));
    sub[lane] = ~(uint32_t)x;
}

// The same with exact scores (the forward's path): the list holds the exact
// top k and their exact scores.
template <int J, bool BF16, bool LAT = false, class SC = float>
__device__ __forceinline__ void select_half_exact(const SC* s, int S, int k, int lane, uint64_t* buf, float* val,
                                                  uint32_t* sub, Refine ref)
{
    const uint64_t x = half_sorted_topk_exact<J, BF16, LAT, SC>(s, S, k, lane, buf, ref);
    val[lane] = key_value((uint32_t)(x >> 32));
    sub[lane] = ~(uint32_t)x;
}

// The W winners in lane order (lane 0 the best) as slots and weights: a softmax
// over their sums in double, each weight rounded once to float32.
__device__ __forceinline__ void emit_winners(uint64_t x, int W, int lane, int32_t* idx_row, float* wt_row)
{
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

// Step 2 by one wave, from both halves' sorted lists (val, sub: 2 x 64, in
// LDS and visible to the wave): idx_row, wt_row receive the W slots and
// weights, best first.  buf: 64 entries of the wave's LDS scratch.  LAT: the
// counting sort.
template <int R, bool LAT = false>
__device__ __forceinline__ void select_from_lists(int S, int k, int W, int n_pairs, const uint16_t* s_pairs, int lane,
                                         uint64_t* buf, const float (*val)[64], const uint32_t (*sub)[64],
                                         int32_t* idx_row, float* wt_row);

// The selection of one row by one wave: s holds the row's half scores (S of
// half 0, then S of half 1; global or LDS); buf, val, sub are the wave's LDS
// scratch (64 entries each, val and sub 2 x 64); idx_row, wt_row receive the W
// slots and weights, best first.
template <int J, int R>
__device__ __forceinline__ void select_row(const float* s, int S, int k, int W, int n_pairs, const uint16_t* s_pairs,
                                  int lane, uint64_t* buf, float (*val)[64], uint32_t (*sub)[64],
                                  int32_t* idx_row, float* wt_row)
{
#pragma unroll
    for (int h = 0; h < 2; ++h)
        select_half<J>(s + h * S, S, k, lane, buf, val[h], sub[h]);
    wave_sync_lds();
    select_from_lists<R>(S, k, W, n_pairs, s_pairs, lane, buf, val, sub, idx_row, wt_row);
}

// select_row with exact scores: ref0, ref1 for halves 0 and 1.
template <int J, int R, bool BF16, bool LAT = false, class SC = float>
__device__ __forceinline__ void select_row_exact(const SC* s, int S, int k, int W, int n_pairs,
                                                 const uint16_t* s_pairs, int lane, uint64_t* buf, float (*val)[64],
                                                 uint32_t (*sub)[64], int32_t* idx_row, float* wt_row, Refine ref0,
                                                 Refine ref1)
{
    select_half_exact<J, BF16, LAT, SC>(s, S, k, lane, buf, val[0], sub[0], ref0);
    select_half_exact<J, BF16, LAT, SC>(s + S, S, k, lane, buf, val[1], sub[1], ref1);
    wave_sync_lds();
    select_from_lists<R, LAT>(S, k, W, n_pairs, s_pairs, lane, buf, val, sub, idx_row, wt_row);
}

// select_row_exact from candidate records (rec0, rec1 for halves 0 and 1).
template <int J, int R, bool BF16>
__device__ __forceinline__ void select_row_cand(const uint32_t* rec0, const uint32_t* rec1, int S, int k, int W,
                                                int n_pairs, const uint16_t* s_pairs, int lane, uint64_t* buf,
                                                float (*val)[64], uint32_t (*sub)[64], int32_t* idx_row,
                                                float* wt_row, Refine ref0, Refine ref1)
{
    const uint32_t* rec[2] = {rec0, rec1};
    const Refine ref[2] = {ref0, ref1};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const uint64_t x = half_sorted_topk_cand<J, BF16>(rec[hf], S, k, lane, buf, ref[hf]);
        val[hf][lane] = key_value((uint32_t)(x >> 32));
        sub[hf][lane] = ~(uint32_t)x;
    }
    wave_sync_lds();
    select_from_lists<R, false>(S, k, W, n_pairs, s_pairs, lane, buf, val, sub, idx_row, wt_row);
}

template <int R, bool LAT>
__device__ __forceinline__ void select_from_lists(int S, int k, int W, int n_pairs, const uint16_t* s_pairs, int lane,
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
    const uint64_t x = lane < W ? buf[lane] : 0ull;
    emit_winners(LAT ? sort64_desc_count(x, lane, buf) : sort64_desc(x, lane), W, lane, idx_row, wt_row);
}

} // namespace pksel
} // namespace sdm
