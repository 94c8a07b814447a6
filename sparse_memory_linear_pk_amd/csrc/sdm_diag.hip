// sdm_overlap: the write/read bucket-overlap diagnostic of the SDM blog post's
// needle-in-a-haystack figure (section "Memory Access Patterns on a
// Needle-in-a-Haystack Task": cumulative writes over the memory's slots, the
// current token's reads, and whether the slots written at the needle are the
// ones read at the query), computed from a call's addressing.
//
//   bucket(n) = n * K / N (a contiguous range of slots; with K = S the first sub-key)
//   write_cum[b, h, t, k] = sum over tokens t' <= t and write positions i with
//                           bucket(n_i(t')) = k of w_i(t')
//   read[b, h, t, k]      = sum over read positions j of token t with bucket k of r_j(t)
//   overlap[b, h, q, a]   = sum over slots n written by token a and read by
//                           query token queries[q] of w_a(n) r_q(n), for a <= queries[q]
//
// bucket_scan_kernel: a thread per bucket walks the tokens in order, adding in
// double in token and position order (so each value is the exactly ordered sum,
// rounded once), with the slot lists of 32 tokens at a time staged in LDS.
// overlap_kernel: a workgroup per (memory, query) holds the query's read slots
// in LDS; a wave per earlier token matches its write slots against them.
#include "sdm_internal.h"

namespace sdm {
namespace {

constexpr int kTok = 32; // tokens staged per round

struct DiagArgs {
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    float* write_cum;
    float* read;
    const int32_t* queries;
    float* overlap;
    int B, T, H, W, K, Q;
    long N;
};

__global__ __launch_bounds__(256) void bucket_scan_kernel(DiagArgs a)
{
    __shared__ int32_t s_nw[kTok * 64], s_nr[kTok * 64]; // buckets of the staged tokens' slots
    __shared__ float s_ww[kTok * 64], s_wr[kTok * 64];
    const int nkb = (a.K + 255) / 256;
    const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    const int b = bh / a.H, h = bh % a.H;
    const int k = kb * 256 + (int)threadIdx.x;
    double acc = 0.0;
    for (int t0 = 0; t0 < a.T; t0 += kTok) {
        const int nt = min(kTok, a.T - t0);
        __syncthreads(); // the previous round's reads are done
        for (int e = threadIdx.x; e < nt * a.W; e += 256) {
            const int tt = e / a.W, i = e % a.W;
            const size_t r = ((size_t)b * a.T + t0 + tt) * a.H + h;
            // buckets, not slots: the division is done once per entry, not once per bucket thread
            s_nw[tt * 64 + i] = (int32_t)((long)a.idx_w[r * a.W + i] * a.K / a.N);
            s_ww[tt * 64 + i] = a.wt_w[r * a.W + i];
            s_nr[tt * 64 + i] = (int32_t)((long)a.idx_r[r * a.W + i] * a.K / a.N);
            s_wr[tt * 64 + i] = a.wt_r[r * a.W + i];
        }
        __syncthreads();
        if (k >= a.K)
            continue; // no barrier skipped: the next one is at the top of the loop, reached by all
        for (int tt = 0; tt < nt; ++tt) {
            double cur = 0.0;
            for (int i = 0; i < a.W; ++i) {
                if (s_nw[tt * 64 + i] == k)
                    acc += (double)s_ww[tt * 64 + i];
                if (s_nr[tt * 64 + i] == k)
                    cur += (double)s_wr[tt * 64 + i];
            }
            const size_t o = (((size_t)b * a.H + h) * a.T + t0 + tt) * a.K + k;
            a.write_cum[o] = (float)acc;
            a.read[o] = (float)cur;
        }
    }
}

__global__ __launch_bounds__(256) void overlap_kernel(DiagArgs a)
{
    __shared__ int32_t s_m[64];
    __shared__ float s_r[64];
    const int bh = blockIdx.x / a.Q, qi = blockIdx.x % a.Q;
    const int b = bh / a.H, h = bh % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = a.queries[qi];
    const bool valid = q >= 0 && q < a.T;
    if (threadIdx.x < 64) {
        const size_t rq = ((size_t)b * a.T + (valid ? q : 0)) * a.H + h;
        s_m[threadIdx.x] = (valid && (int)threadIdx.x < a.W) ? a.idx_r[rq * a.W + threadIdx.x] : -1;
        s_r[threadIdx.x] = (valid && (int)threadIdx.x < a.W) ? a.wt_r[rq * a.W + threadIdx.x] : 0.f;
    }
    __syncthreads();
    float* out = a.overlap + (((size_t)b * a.H + h) * a.Q + qi) * a.T;
    for (int t = wave; t < a.T; t += 4) {
        double s = 0.0;
        if (valid && t <= q) { // wave-uniform
            const size_t ra = ((size_t)b * a.T + t) * a.H + h;
            const bool live = lane < a.W;
            const int32_t n = live ? a.idx_w[ra * a.W + lane] : -2;
            const double w = live ? (double)a.wt_w[ra * a.W + lane] : 0.0;
            for (int j = 0; j < a.W; ++j)
                if (s_m[j] == n)
                    s += w * (double)s_r[j]; // exact: a product of two floats
#pragma unroll
            for (int o = 1; o < 64; o <<= 1)
                s += __shfl_xor(s, o);
        }
        if (lane == 0)
            out[t] = (float)s;
    }
}

} // namespace

hipError_t launch_overlap(const int32_t* idx_w, const float* wt_w, const int32_t* idx_r, const float* wt_r, int K,
                          float* write_cum, float* read, int Q, const int32_t* queries, float* overlap, int B, int T,
                          int H, int W, long N, hipStream_t stream)
{
    if (K < 1 || K > N || W < 1 || W > 64 || Q < 0)
        return hipErrorInvalidValue;
    DiagArgs a{idx_w, wt_w, idx_r, wt_r, write_cum, read, queries, overlap, B, T, H, W, K, Q, N};
    const int nkb = (K + 255) / 256;
    hipLaunchKernelGGL(bucket_scan_kernel, dim3((unsigned)(B * H * nkb)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || Q == 0)
        return e;
    hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)(B * H * Q)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace sdm
