/*
 * Reference oracle for the Sparse Delta Memory (SDM) layer forward pass.
 * TEST INFRASTRUCTURE: see sdm_oracle.h for who may use it, the layouts and
 * the source of each step.  Plain, slow and sequential on purpose.
 */
#include "sdm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t float_bits_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* bfloat16 keeps 8 significant bits and float32's exponent range.  Round a
 * double straight to it, nearest with ties to even, keeping subnormals
 * (spacing 2^-133) and overflowing to infinity. */
uint16_t oracle_bf16_round(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e); /* a = m * 2^e with m in [0.5, 1) */
    int qexp = e - 8; /* weight of the 8th significant bit */
    if (qexp < -133)
        qexp = -133;
    double q = ldexp(1.0, qexp);
    double r = nearbyint(a / q) * q; /* a / q is exact; default mode is ties-to-even */
    if (r > 0x1.fep127) /* largest finite bfloat16, (2 - 2^-7) * 2^127 */
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | float_bits_hi((float)r));
}

static double load_in(const void* p, size_t i, int bf16)
{
    return bf16 ? bf16_to_double(((const uint16_t*)p)[i]) : (double)((const float*)p)[i];
}

/* State storage kinds: 0 float32, 1 bf16 bits, 2 float64 (no rounding at
 * store; used only to check derivatives by finite differences). */
static double load_state(const void* mem, size_t i, int kind)
{
    if (kind == 2)
        return ((const double*)mem)[i];
    return load_in(mem, i, kind);
}

static void store_state(void* mem, size_t i, double x, int kind)
{
    if (kind == 2)
        ((double*)mem)[i] = x;
    else if (kind)
        ((uint16_t*)mem)[i] = oracle_bf16_round(x);
    else
        ((float*)mem)[i] = (float)x; /* nearest-even */
}

/* ------------------------------------------------------------------------ */
/* ordering: larger value first, then smaller index first                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t i;
} scored;

static int by_value_desc_index_asc(const void* pa, const void* pb)
{
    const scored* a = (const scored*)pa;
    const scored* b = (const scored*)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* ------------------------------------------------------------------------ */
/* product-key addressing                                                    */
/* ------------------------------------------------------------------------ */

static int cfg_ok(const oracle_cfg* c)
{
    return c && c->B > 0 && c->H > 0 && c->T > 0 && c->d > 0 && c->S > 0 && c->dk > 0 &&
           c->dk % 2 == 0 && c->k > 0 && c->k <= c->S && c->W > 0 && (long)c->W <= (long)c->k * c->k;
}

/* The two score sets: the first half of the query against sub-key table 0 and
 * the second half against table 1 ("two sub-keys" in the figure caption).
 * Each is a dot product, accumulated in double and rounded once to float. */
int oracle_scores(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                  float* scores)
{
    if (!cfg_ok(c) || !q || !subkeys || !scores || row0 < 0 || row1 > (long)c->B * c->T * c->H)
        return -1;
    const int S = c->S, dh = c->dk / 2;
    for (long r = row0; r < row1; ++r) {
        int h = (int)(r % c->H);
        for (int half = 0; half < 2; ++half) {
            for (int i = 0; i < S; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dh; ++j) {
                    double qj = load_in(q, (size_t)r * c->dk + (size_t)half * dh + j, c->in_bf16);
                    double kj = load_in(subkeys, (((size_t)h * 2 + half) * S + i) * dh + j, c->in_bf16);
                    acc += qj * kj;
                }
                scores[((size_t)(r - row0) * 2 + half) * S + i] = (float)acc;
            }
        }
    }
    return 0;
}

int oracle_topk(const float* s, int n, int k, int32_t* idx)
{
    if (!s || !idx || n <= 0 || k <= 0 || k > n)
        return -1;
    scored* all = (scored*)malloc(sizeof(scored) * (size_t)n);
    if (!all)
        return -1;
    for (int i = 0; i < n; ++i) {
        all[i].v = s[i];
        all[i].i = i;
    }
    qsort(all, (size_t)n, sizeof(scored), by_value_desc_index_asc);
    for (int i = 0; i < k; ++i)
        idx[i] = all[i].i;
    free(all);
    return 0;
}

/* Per-half top-k, then every pair (a, b) of survivors is a candidate slot
 * n = a*S + b whose score is the float sum s1[a] + s2[b] ("outer sum" in the
 * figure caption); the W best candidates are kept. */
int oracle_select(const float* s1, const float* s2, int S, int k, int W, int32_t* slot, float* sigma)
{
    if (!s1 || !s2 || !slot || !sigma || k <= 0 || k > S || W <= 0 || (long)W > (long)k * k)
        return -1;
    int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t* b = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)k * k);
    int rc = -1;
    if (!a || !b || !cand)
        goto done;
    if (oracle_topk(s1, S, k, a) || oracle_topk(s2, S, k, b))
        goto done;
    for (int i = 0; i < k; ++i) {
        for (int j = 0; j < k; ++j) {
            float sum = s1[a[i]] + s2[b[j]]; /* one float addition */
            cand[(size_t)i * k + j].v = sum;
            cand[(size_t)i * k + j].i = a[i] * S + b[j];
        }
    }
    qsort(cand, (size_t)k * k, sizeof(scored), by_value_desc_index_asc);
    for (int i = 0; i < W; ++i) {
        slot[i] = cand[i].i;
        sigma[i] = cand[i].v;
    }
    rc = 0;
done:
    free(a);
    free(b);
    free(cand);
    return rc;
}

/* Softmax over the W selected sums (the caption names a softmax-weighted
 * read; the same weights are taken for the write, with no temperature). */
int oracle_softmax(const float* sigma, int W, float* w)
{
    if (!sigma || !w || W <= 0)
        return -1;
    double m = sigma[0];
    for (int i = 1; i < W; ++i)
        if (sigma[i] > m)
            m = sigma[i];
    double z = 0.0;
    for (int i = 0; i < W; ++i)
        z += exp((double)sigma[i] - m);
    for (int i = 0; i < W; ++i)
        w[i] = (float)(exp((double)sigma[i] - m) / z);
    return 0;
}

int oracle_address_from_scores(const oracle_cfg* c, const float* scores, long row0, long row1,
                               int32_t* idx, float* wt, float* sigma)
{
    if (!cfg_ok(c) || !scores || !idx || !wt || row0 < 0 || row1 > (long)c->B * c->T * c->H)
        return -1;
    const int S = c->S, W = c->W;
    float* sg = sigma ? NULL : (float*)malloc(sizeof(float) * (size_t)W);
    for (long r = row0; r < row1; ++r) {
        size_t o = (size_t)(r - row0);
        const float* s1 = scores + (o * 2 + 0) * S;
        const float* s2 = scores + (o * 2 + 1) * S;
        float* sig = sigma ? sigma + o * W : sg;
        if (!sig || oracle_select(s1, s2, S, c->k, W, idx + o * W, sig) ||
            oracle_softmax(sig, W, wt + o * W)) {
            free(sg);
            return -1;
        }
    }
    free(sg);
    return 0;
}

int oracle_address(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                   int32_t* idx, float* wt, float* sigma)
{
    if (!cfg_ok(c) || row0 < 0 || row1 < row0)
        return -1;
    const int S = c->S;
    float* sc = (float*)malloc(sizeof(float) * 2 * (size_t)S);
    float* sg = (float*)malloc(sizeof(float) * (size_t)c->W);
    if (!sc || !sg) {
        free(sc);
        free(sg);
        return -1;
    }
    int rc = 0;
    for (long r = row0; r < row1 && rc == 0; ++r) {
        size_t o = (size_t)(r - row0);
        rc = oracle_scores(c, q, subkeys, r, r + 1, sc);
        if (rc == 0)
            rc = oracle_select(sc, sc + S, S, c->k, c->W, idx + o * c->W, sigma ? sigma + o * c->W : sg);
        if (rc == 0)
            rc = oracle_softmax(sigma ? sigma + o * c->W : sg, c->W, wt + o * c->W);
    }
    free(sc);
    free(sg);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* the memory scan                                                           */
/* ------------------------------------------------------------------------ */

/* One token t of memory (b, h), with write slots n_i, weights w_i, decay a,
 * step size beta, value v and read slots m_j, weights r_j:
 *   x_i   = a * M[n_i]                 decay of the write-selected slots only
 *   vhat  = sum_i w_i x_i              the memory's prediction of v
 *   delta = beta * (v - vhat)
 *   M[n_i] = store(x_i + w_i * delta)  delta-rule write
 *   out   = sum_j r_j M[m_j]           read of the stored values, after the write
 * This is the gated delta rule with the key taken as the sparse weight vector
 * and the decay confined to the selected slots: the SDM blog post's section
 * "How does SDM work?" and the caption of its figure "The SDM mechanism, end
 * to end" order the write as a decay of the chosen slots followed by a
 * delta-rule update toward v.  Slots not selected are left as they are. */
int oracle_scan(const oracle_cfg* c, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                const float* wt_r, const void* v, const float* alpha, const float* beta, void* mem,
                float* out, int b, int h, int e0, int e1)
{
    if (!cfg_ok(c) || !idx_w || !wt_w || !idx_r || !wt_r || !v || !alpha || !beta || !mem || !out ||
        b < 0 || b >= c->B || h < 0 || h >= c->H || e0 < 0 || e1 > c->d || e0 >= e1)
        return -1;
    const int W = c->W, d = c->d, ne = e1 - e0;
    const size_t N = (size_t)c->S * c->S;
    const size_t base = ((size_t)b * c->H + h) * N; /* first slot of memory (b, h) */
    double* x = (double*)malloc(sizeof(double) * (size_t)W * ne);
    double* delta = (double*)malloc(sizeof(double) * (size_t)ne);
    if (!x || !delta) {
        free(x);
        free(delta);
        return -1;
    }
    for (int t = 0; t < c->T; ++t) {
        const size_t r = ((size_t)b * c->T + t) * c->H + h;
        const int32_t* n = idx_w + r * W;
        const float* w = wt_w + r * W;
        const int32_t* m = idx_r + r * W;
        const float* rw = wt_r + r * W;
        const double a = alpha[r], be = beta[r];
        for (int i = 0; i < W; ++i) {
            if (n[i] < 0 || (size_t)n[i] >= N)
                goto bad;
            for (int e = 0; e < ne; ++e)
                x[(size_t)i * ne + e] = a * load_state(mem, (base + n[i]) * d + e0 + e, c->state_bf16);
        }
        for (int e = 0; e < ne; ++e) {
            double vhat = 0.0;
            for (int i = 0; i < W; ++i)
                vhat += (double)w[i] * x[(size_t)i * ne + e];
            delta[e] = be * (load_in(v, r * d + e0 + e, c->in_bf16) - vhat);
        }
        for (int i = 0; i < W; ++i)
            for (int e = 0; e < ne; ++e)
                store_state(mem, (base + n[i]) * d + e0 + e,
                            x[(size_t)i * ne + e] + (double)w[i] * delta[e], c->state_bf16);
        for (int e = 0; e < ne; ++e) {
            double o = 0.0;
            for (int j = 0; j < W; ++j) {
                if (m[j] < 0 || (size_t)m[j] >= N)
                    goto bad;
                o += (double)rw[j] * load_state(mem, (base + m[j]) * d + e0 + e, c->state_bf16);
            }
            out[r * d + e0 + e] = (float)o;
        }
    }
    free(x);
    free(delta);
    return 0;
bad:
    free(x);
    free(delta);
    return -1;
}
