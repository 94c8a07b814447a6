/*
 * Reference oracle for the write/read bucket-overlap diagnostic.
 * TEST INFRASTRUCTURE (see sdm_oracle_proj.h): plain and sequential.
 *
 * The SDM blog post's needle-in-a-haystack figure (section "Memory Access
 * Patterns on a Needle-in-a-Haystack Task") shows, per token, the cumulative
 * writes over the memory's slots, the current token's reads, and whether the
 * slots written at the needle are the ones read at the query.  Readings: a
 * bucket is a contiguous range of slots, bucket(n) = n * K / N (with K = S it
 * is the first sub-key of the slot); a bucket's write mass is the sum of the
 * write weights of its selected slots, accumulated over the tokens up to and
 * including t; its read mass is the current token's read weights; the overlap
 * of write token a and read token q is the sum over the slots both select of
 * w_a(n) * r_q(n), for a <= q (the write of token q itself comes before its
 * read), zero for a > q.
 *
 * Layouts: idx, wt [B*T*H, W] as the forward's addressing (row (b*T + t)*H + h);
 * write_cum, read [B, H, T, K] float32; queries [Q] token indices;
 * overlap [B, H, Q, T] float32.  Sums in double, rounded once.
 */
#include <stdint.h>
#include <stdlib.h>

int oracle_overlap(int B, int T, int H, int W, long N, int K, const int32_t* idx_w, const float* wt_w,
                   const int32_t* idx_r, const float* wt_r, int Q, const int32_t* queries, float* write_cum,
                   float* read, float* overlap)
{
    if (B < 1 || T < 1 || H < 1 || W < 1 || N < 1 || K < 1 || K > N || Q < 0 || !idx_w || !wt_w || !idx_r ||
        !wt_r || !write_cum || !read || (Q > 0 && (!queries || !overlap)))
        return -1;
    double* acc = (double*)calloc((size_t)K, sizeof(double));
    double* cur = (double*)calloc((size_t)K, sizeof(double));
    if (!acc || !cur) {
        free(acc);
        free(cur);
        return -1;
    }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            for (int k = 0; k < K; ++k)
                acc[k] = 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t r = ((size_t)b * T + t) * H + h;
                for (int k = 0; k < K; ++k)
                    cur[k] = 0.0;
                for (int i = 0; i < W; ++i) {
                    const int32_t nw = idx_w[r * W + i], nr = idx_r[r * W + i];
                    if (nw < 0 || nw >= N || nr < 0 || nr >= N) {
                        free(acc);
                        free(cur);
                        return -1;
                    }
                    acc[(long)nw * K / N] += wt_w[r * W + i];
                    cur[(long)nr * K / N] += wt_r[r * W + i];
                }
                float* wc = write_cum + (((size_t)b * H + h) * T + t) * K;
                float* rd = read + (((size_t)b * H + h) * T + t) * K;
                for (int k = 0; k < K; ++k) {
                    wc[k] = (float)acc[k];
                    rd[k] = (float)cur[k];
                }
            }
            for (int qi = 0; qi < Q; ++qi) {
                const int q = queries[qi];
                if (q < 0 || q >= T) {
                    free(acc);
                    free(cur);
                    return -1;
                }
                const size_t rq = ((size_t)b * T + q) * H + h;
                float* o = overlap + (((size_t)b * H + h) * Q + qi) * T;
                for (int a = 0; a < T; ++a) {
                    double s = 0.0;
                    if (a <= q) {
                        const size_t ra = ((size_t)b * T + a) * H + h;
                        for (int i = 0; i < W; ++i)
                            for (int j = 0; j < W; ++j)
                                if (idx_w[ra * W + i] == idx_r[rq * W + j])
                                    s += (double)wt_w[ra * W + i] * wt_r[rq * W + j];
                    }
                    o[a] = (float)s;
                }
            }
        }
    free(acc);
    free(cur);
    return 0;
}
