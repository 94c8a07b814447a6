/*
 * Runs every oracle routine on small seeded inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/sanitize/build.py): float32 and
 * bf16 inputs, float32, bf16 and float64 states, the edge shapes (one token,
 * k = S, W = k*k, W = 1), every rejected argument, and the gradient,
 * projection and bucket-overlap routines.  Exits 0 when every call returned
 * what it should; a sanitizer report aborts the run.  Test code only.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sdm_oracle.h"
#include "sdm_oracle_grad.h"
#include "sdm_oracle_proj.h"

int oracle_overlap(int B, int T, int H, int W, long N, int K, const int32_t* idx_w, const float* wt_w,
                   const int32_t* idx_r, const float* wt_r, int Q, const int32_t* queries, float* write_cum,
                   float* read, float* overlap);

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) /* splitmix64 */
{
    unsigned long long z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1p-53;
}

static double normal(void) { return sqrt(-2.0 * log(uniform() + 1e-300)) * cos(6.283185307179586 * uniform()); }

static int failures = 0;

#define EXPECT(cond)                                                                                             \
    do {                                                                                                         \
        if (!(cond)) {                                                                                           \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond);                       \
            ++failures;                                                                                          \
        }                                                                                                        \
    } while (0)

static void* fill_in(size_t n, int bf16, double std)
{
    void* p = malloc(n * (bf16 ? 2 : 4));
    for (size_t i = 0; i < n; ++i) {
        const double x = normal() * std;
        if (bf16)
            ((uint16_t*)p)[i] = oracle_bf16_round(x);
        else
            ((float*)p)[i] = (float)x;
    }
    return p;
}

static void* fill_state(size_t n, int kind, double std)
{
    const size_t es = kind == 2 ? 8 : kind == 1 ? 2 : 4;
    void* p = malloc(n * es);
    for (size_t i = 0; i < n; ++i) {
        const double x = normal() * std;
        if (kind == 2)
            ((double*)p)[i] = x;
        else if (kind == 1)
            ((uint16_t*)p)[i] = oracle_bf16_round(x);
        else
            ((float*)p)[i] = (float)x;
    }
    return p;
}

/* Addressing, scan and gradients of one configuration. */
static void run_config(oracle_cfg c)
{
    const long R = (long)c.B * c.T * c.H;
    const size_t N = (size_t)c.S * c.S;
    const int dh = c.dk / 2;
    void* wq = fill_in((size_t)R * c.dk, c.in_bf16, 1.0);
    void* rq = fill_in((size_t)R * c.dk, c.in_bf16, 1.0);
    void* v = fill_in((size_t)R * c.d, c.in_bf16, 1.0);
    void* sk = fill_in((size_t)c.H * 2 * c.S * dh, c.in_bf16, 0.25);
    float* alpha = malloc(R * sizeof(float));
    float* beta = malloc(R * sizeof(float));
    for (long r = 0; r < R; ++r) {
        alpha[r] = (float)(1.0 / (1.0 + exp(-(normal() + 2.0))));
        beta[r] = (float)(1.0 / (1.0 + exp(-normal())));
    }
    float* scores = malloc(R * 2 * c.S * sizeof(float));
    int32_t* iw = malloc(R * c.W * sizeof(int32_t));
    int32_t* ir = malloc(R * c.W * sizeof(int32_t));
    int32_t* i2 = malloc(R * c.W * sizeof(int32_t));
    float* ww = malloc(R * c.W * sizeof(float));
    float* wr = malloc(R * c.W * sizeof(float));
    float* w2 = malloc(R * c.W * sizeof(float));
    float* sg = malloc(R * c.W * sizeof(float));
    EXPECT(oracle_scores(&c, wq, sk, 0, R, scores) == 0);
    EXPECT(oracle_address(&c, wq, sk, 0, R, iw, ww, sg) == 0);
    EXPECT(oracle_address(&c, rq, sk, 0, R, ir, wr, NULL) == 0);
    EXPECT(oracle_address_from_scores(&c, scores, 0, R, i2, w2, NULL) == 0);
    EXPECT(memcmp(iw, i2, R * c.W * sizeof(int32_t)) == 0 && memcmp(ww, w2, R * c.W * sizeof(float)) == 0);
    for (long j = 0; j < R * c.W; ++j)
        EXPECT(iw[j] >= 0 && (size_t)iw[j] < N && isfinite(ww[j]));
    for (int kind = 0; kind <= 2; ++kind) {
        oracle_cfg cs = c;
        cs.state_bf16 = kind;
        void* mem = fill_state((size_t)c.B * c.H * N * c.d, kind, 0.05);
        float* out = malloc(R * c.d * sizeof(float));
        for (int b = 0; b < c.B; ++b)
            for (int h = 0; h < c.H; ++h) {
                EXPECT(oracle_scan(&cs, iw, ww, ir, wr, v, alpha, beta, mem, out, b, h, 0, c.d) == 0);
                if (c.d > 2) /* a slice of the elements as well */
                    EXPECT(oracle_scan(&cs, iw, ww, ir, wr, v, alpha, beta, mem, out, b, h, 1, c.d - 1) == 0);
            }
        for (long j = 0; j < R * c.d; ++j)
            EXPECT(isfinite(out[j]));
        free(out);
        free(mem);
    }
    /* gradients (float32 state) */
    {
        void* mem0 = fill_state((size_t)c.B * c.H * N * c.d, 0, 0.05);
        float* dout = (float*)fill_in((size_t)R * c.d, 0, 1.0);
        double* dmem = calloc((size_t)c.B * c.H * N * c.d, sizeof(double));
        double* dv = calloc((size_t)R * c.d, sizeof(double));
        double* dal = calloc(R, sizeof(double));
        double* dbe = calloc(R, sizeof(double));
        double* dww = calloc((size_t)R * c.W, sizeof(double));
        double* dwr = calloc((size_t)R * c.W, sizeof(double));
        for (int b = 0; b < c.B; ++b)
            for (int h = 0; h < c.H; ++h)
                EXPECT(oracle_scan_grad(&c, iw, ww, ir, wr, v, alpha, beta, mem0, dout, dmem, dv, dal, dbe, dww, dwr,
                                        b, h) == 0);
        double* dq = calloc((size_t)R * c.dk, sizeof(double));
        double* dsub = calloc((size_t)c.H * 2 * c.S * dh, sizeof(double));
        EXPECT(oracle_address_grad(&c, wq, sk, 0, R, iw, sg, dww, dq, dsub) == 0);
        double* q64 = malloc(c.dk * sizeof(double));
        double* sk64 = malloc((size_t)c.H * 2 * c.S * dh * sizeof(double));
        for (int j = 0; j < c.dk; ++j)
            q64[j] = normal();
        for (size_t j = 0; j < (size_t)c.H * 2 * c.S * dh; ++j)
            sk64[j] = normal() * 0.25;
        double* w64 = malloc(c.W * sizeof(double));
        EXPECT(oracle_weights_f64(&c, q64, sk64, c.H - 1, iw, w64) == 0);
        free(mem0), free(dout), free(dmem), free(dv), free(dal), free(dbe), free(dww), free(dwr), free(dq);
        free(dsub), free(q64), free(sk64), free(w64);
    }
    /* bucket overlap */
    {
        const int K = c.S, Q = 2;
        int32_t qs[2] = {0, c.T - 1};
        float* wc = malloc((size_t)R * K * sizeof(float));
        float* rd = malloc((size_t)R * K * sizeof(float));
        float* ov = malloc((size_t)c.B * c.H * Q * c.T * sizeof(float));
        EXPECT(oracle_overlap(c.B, c.T, c.H, c.W, (long)N, K, iw, ww, ir, wr, Q, qs, wc, rd, ov) == 0);
        free(wc), free(rd), free(ov);
    }
    free(wq), free(rq), free(v), free(sk), free(alpha), free(beta), free(scores);
    free(iw), free(ir), free(i2), free(ww), free(wr), free(w2), free(sg);
}

int main(void)
{
    const oracle_cfg cfgs[] = {
        {1, 1, 9, 8, 8, 16, 3, 5, 0, 0},    /* small float32 */
        {2, 3, 5, 16, 6, 32, 4, 12, 1, 0},  /* bf16 inputs, several heads and sequences */
        {1, 1, 1, 4, 5, 16, 5, 25, 0, 0},   /* one token, k = S, W = k*k */
        {1, 2, 7, 3, 9, 16, 1, 1, 1, 0},    /* k = W = 1, odd width */
        {1, 1, 12, 8, 40, 64, 8, 64, 1, 0}, /* W = 64 */
    };
    for (size_t i = 0; i < sizeof cfgs / sizeof cfgs[0]; ++i)
        run_config(cfgs[i]);

    /* rejected arguments */
    oracle_cfg c = cfgs[0];
    float s[8] = {0};
    int32_t idx[8];
    float w[8], sig[8];
    EXPECT(oracle_topk(s, 8, 9, idx) != 0);
    EXPECT(oracle_topk(NULL, 8, 2, idx) != 0);
    EXPECT(oracle_select(s, s, 8, 9, 4, idx, sig) != 0);
    EXPECT(oracle_select(s, s, 8, 2, 5, idx, sig) != 0);
    EXPECT(oracle_softmax(sig, 0, w) != 0);
    oracle_cfg bad = c;
    bad.k = c.S + 1;
    EXPECT(oracle_scores(&bad, s, s, 0, 1, s) != 0);
    bad = c;
    bad.dk = 15;
    EXPECT(oracle_address(&bad, s, s, 0, 1, idx, w, sig) != 0);
    EXPECT(oracle_scores(&c, s, s, 0, (long)c.B * c.T * c.H + 1, s) != 0);
    EXPECT(oracle_scan(&c, idx, w, idx, w, s, s, s, s, s, 0, 0, 3, 2) != 0);
    EXPECT(oracle_scan(&c, idx, w, idx, w, s, s, s, s, s, 1, 0, 0, 1) != 0);
    EXPECT(oracle_overlap(1, 1, 1, 1, 4, 5, idx, w, idx, w, 0, NULL, w, w, NULL) != 0);
    /* projection and broadcast */
    {
        const int B = 2, T = 3, H = 2, D = 24, dk = 8, d = 8, C = 2 * dk + d + 2;
        uint16_t* x = fill_in((size_t)B * T * D, 1, 1.0);
        uint16_t* wp = fill_in((size_t)H * C * D, 1, 0.2);
        float bias[4] = {4.f, 0.f, 3.f, -1.f};
        uint16_t* wq = malloc((size_t)B * T * H * dk * 2);
        uint16_t* rq = malloc((size_t)B * T * H * dk * 2);
        uint16_t* v = malloc((size_t)B * T * H * d * 2);
        float* al = malloc((size_t)B * T * H * 4);
        float* be = malloc((size_t)B * T * H * 4);
        EXPECT(oracle_project(B, T, H, D, dk, d, x, wp, bias, 0, B * T, wq, rq, v, al, be) == 0);
        EXPECT(oracle_project(B, T, H, D, dk, d, x, wp, bias, 0, B * T + 1, wq, rq, v, al, be) != 0);
        float m0[2 * 6], mem[3 * 2 * 6];
        for (int i = 0; i < 12; ++i)
            m0[i] = (float)i;
        EXPECT(oracle_broadcast_memory(3, 2, 6 * sizeof(float), m0, mem) == 0);
        EXPECT(mem[2 * 12 + 11] == 11.f);
        free(x), free(wp), free(wq), free(rq), free(v), free(al), free(be);
    }
    if (failures)
        fprintf(stderr, "%d expectations failed\n", failures);
    else
        printf("oracle checks ok\n");
    return failures ? 1 : 0;
}
