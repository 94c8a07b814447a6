/*
 * Reference oracle for the SDM layer's backward pass.
 * TEST INFRASTRUCTURE: see sdm_oracle_grad.h for who may use it, what is
 * differentiated and the readings taken.  Plain, slow and sequential.
 */
#include "sdm_oracle_grad.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double in_value(const void* p, size_t i, int bf16)
{
    if (bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    return ((const float*)p)[i];
}

static size_t state_size(int kind) { return kind == 2 ? 8 : kind == 1 ? 2 : 4; }

static double state_value(const void* mem, size_t i, int kind)
{
    if (kind == 2)
        return ((const double*)mem)[i];
    return in_value(mem, i, kind);
}

/* ------------------------------------------------------------------------ */
/* the scan                                                                  */
/* ------------------------------------------------------------------------ */

/* Forward of one token (sdm_oracle.c, oracle_scan), with write slots n_i,
 * weights w_i, decay a, step size beta, value v, read slots m_j, weights r_j:
 *   x_i = a M[n_i],  vhat = sum_i w_i x_i,  delta = beta (v - vhat),
 *   M[n_i] <- x_i + w_i delta,  out = sum_j r_j M[m_j]  (after the write).
 * Its reverse, given G = dL/dM after the token and dout:
 *   read:   dr_j = <dout, M[m_j]>;  G[m_j] += r_j dout
 *   write:  g_i = G[n_i];  ddelta = sum_i w_i g_i;  dv = beta ddelta;
 *           dbeta = <ddelta, v - vhat>;  dvhat = -beta ddelta;
 *           dw_i = <g_i, delta> + <dvhat, x_i>;  dx_i = g_i + w_i dvhat;
 *           da = sum_i <dx_i, M_old[n_i]>;  G[n_i] = a dx_i
 * The read comes first because in the forward it follows the write; a slot
 * both written and read therefore passes its read gradient into the write. */
int oracle_scan_grad(const oracle_cfg* c, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                     const float* wt_r, const void* v, const float* alpha, const float* beta, const void* mem0,
                     const float* dout, double* dmem, double* dv, double* dalpha, double* dbeta, double* dwt_w,
                     double* dwt_r, int b, int h)
{
    if (!c || !idx_w || !wt_w || !idx_r || !wt_r || !v || !alpha || !beta || !mem0 || !dout || !dmem || !dv ||
        !dalpha || !dbeta || !dwt_w || !dwt_r || b < 0 || b >= c->B || h < 0 || h >= c->H || c->T <= 0 ||
        c->d <= 0 || c->W <= 0 || c->S <= 0 || c->state_bf16 < 0 || c->state_bf16 > 2)
        return -1;
    const int T = c->T, W = c->W, d = c->d, kind = c->state_bf16;
    const size_t N = (size_t)c->S * c->S, ssz = state_size(kind), insz = c->in_bf16 ? 2 : 4;
    const size_t base = ((size_t)b * c->H + h) * N;
    for (long r = 0; r < (long)c->B * T * c->H; ++r)
        for (int i = 0; i < W; ++i)
            if (idx_w[r * W + i] < 0 || (size_t)idx_w[r * W + i] >= N || idx_r[r * W + i] < 0 ||
                (size_t)idx_r[r * W + i] >= N)
                return -1;

    unsigned char* work = (unsigned char*)malloc(N * d * ssz);
    double* wlog = (double*)malloc(sizeof(double) * (size_t)T * W * d);
    double* g = (double*)malloc(sizeof(double) * (size_t)W * d);
    double* x = (double*)malloc(sizeof(double) * (size_t)W * d);
    double* vhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* delta = (double*)malloc(sizeof(double) * (size_t)d);
    double* ddelta = (double*)malloc(sizeof(double) * (size_t)d);
    float* tmp_out = (float*)malloc(sizeof(float) * (size_t)d);
    int rc = -1;
    if (!work || !wlog || !g || !x || !vhat || !delta || !ddelta || !tmp_out)
        goto done;
    memcpy(work, (const unsigned char*)mem0 + base * d * ssz, N * d * ssz);

    /* replay the forward one token at a time, recording each write slot's value before its write */
    oracle_cfg one = *c;
    one.B = one.H = one.T = 1;
    for (int t = 0; t < T; ++t) {
        const size_t r = ((size_t)b * T + t) * c->H + h;
        const int32_t* n = idx_w + r * W;
        for (int i = 0; i < W; ++i)
            for (int e = 0; e < d; ++e)
                wlog[((size_t)t * W + i) * d + e] = state_value(work, (size_t)n[i] * d + e, kind);
        if (oracle_scan(&one, n, wt_w + r * W, idx_r + r * W, wt_r + r * W, (const unsigned char*)v + r * d * insz,
                        alpha + r, beta + r, work, tmp_out, 0, 0, 0, d))
            goto done;
    }

    /* the reverse walk */
    double* G = dmem + base * d;
    for (int t = T - 1; t >= 0; --t) {
        const size_t r = ((size_t)b * T + t) * c->H + h;
        const int32_t* n = idx_w + r * W;
        const int32_t* m = idx_r + r * W;
        const float* w = wt_w + r * W;
        const float* rw = wt_r + r * W;
        const float* go = dout + r * d;
        const double a = alpha[r], be = beta[r];

        /* read: the memory now holds its state after token t's write */
        for (int j = 0; j < W; ++j) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e)
                acc += (double)go[e] * state_value(work, (size_t)m[j] * d + e, kind);
            dwt_r[r * W + j] = acc;
            for (int e = 0; e < d; ++e)
                G[(size_t)m[j] * d + e] += (double)rw[j] * (double)go[e];
        }

        /* write: recompute the forward's decayed values, prediction and delta */
        for (int i = 0; i < W; ++i)
            for (int e = 0; e < d; ++e) {
                x[(size_t)i * d + e] = a * wlog[((size_t)t * W + i) * d + e];
                g[(size_t)i * d + e] = G[(size_t)n[i] * d + e];
            }
        double db = 0.0;
        for (int e = 0; e < d; ++e) {
            double yh = 0.0, dd = 0.0;
            for (int i = 0; i < W; ++i) {
                yh += (double)w[i] * x[(size_t)i * d + e];
                dd += (double)w[i] * g[(size_t)i * d + e];
            }
            const double ve = in_value(v, r * d + e, c->in_bf16);
            vhat[e] = yh;
            delta[e] = be * (ve - yh);
            ddelta[e] = dd;
            dv[r * d + e] = be * dd;
            db += dd * (ve - yh);
        }
        dbeta[r] = db;
        double da = 0.0;
        for (int i = 0; i < W; ++i) {
            double dw = 0.0;
            for (int e = 0; e < d; ++e) {
                const double dvhat = -be * ddelta[e];
                const double gi = g[(size_t)i * d + e];
                dw += gi * delta[e] + dvhat * x[(size_t)i * d + e];
                const double dx = gi + (double)w[i] * dvhat;
                da += dx * wlog[((size_t)t * W + i) * d + e];
                G[(size_t)n[i] * d + e] = a * dx;
            }
            dwt_w[r * W + i] = dw;
        }
        dalpha[r] = da;

        /* restore the write slots to their values before token t */
        for (int i = 0; i < W; ++i)
            for (int e = 0; e < d; ++e) {
                const double old = wlog[((size_t)t * W + i) * d + e];
                const size_t at = (size_t)n[i] * d + e;
                if (kind == 2)
                    ((double*)work)[at] = old;
                else if (kind == 1)
                    ((uint16_t*)work)[at] = oracle_bf16_round(old); /* exact: old is a bf16 value */
                else
                    ((float*)work)[at] = (float)old; /* exact: old is a float value */
            }
    }
    rc = 0;
done:
    free(work);
    free(wlog);
    free(g);
    free(x);
    free(vhat);
    free(delta);
    free(ddelta);
    free(tmp_out);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* addressing                                                                */
/* ------------------------------------------------------------------------ */

int oracle_weights_f64(const oracle_cfg* c, const double* q, const double* subkeys, int h, const int32_t* slot,
                       double* w)
{
    if (!c || !q || !subkeys || !slot || !w || h < 0 || h >= c->H || c->W <= 0 || c->dk <= 0 || c->dk % 2)
        return -1;
    const int S = c->S, dh = c->dk / 2, W = c->W;
    double m = -INFINITY;
    for (int i = 0; i < W; ++i) {
        if (slot[i] < 0 || slot[i] >= S * S)
            return -1;
        const int a = slot[i] / S, bb = slot[i] % S;
        double s = 0.0;
        for (int j = 0; j < dh; ++j)
            s += q[j] * subkeys[(((size_t)h * 2 + 0) * S + a) * dh + j];
        for (int j = 0; j < dh; ++j)
            s += q[dh + j] * subkeys[(((size_t)h * 2 + 1) * S + bb) * dh + j];
        w[i] = s;
        if (s > m)
            m = s;
    }
    double z = 0.0;
    for (int i = 0; i < W; ++i)
        z += exp(w[i] - m);
    for (int i = 0; i < W; ++i)
        w[i] = exp(w[i] - m) / z;
    return 0;
}

/* With w = softmax(sigma): dsigma_i = w_i (dw_i - sum_k w_k dw_k).  sigma_i is
 * the first half's score of sub-key a_i plus the second half's of b_i, each a
 * dot product of a query half with a sub-key row, so
 *   dq[0:dh]  += dsigma_i K0[a_i],   dq[dh:dk] += dsigma_i K1[b_i],
 *   dK0[a_i]  += dsigma_i q[0:dh],   dK1[b_i]  += dsigma_i q[dh:dk]. */
int oracle_address_grad(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                        const int32_t* idx, const float* sigma, const double* dwt, double* dq, double* dsub)
{
    if (!c || !q || !subkeys || !idx || !sigma || !dwt || !dq || !dsub || row0 < 0 || row1 < row0 ||
        row1 > (long)c->B * c->T * c->H || c->W <= 0 || c->dk <= 0 || c->dk % 2)
        return -1;
    const int S = c->S, dh = c->dk / 2, W = c->W, dk = c->dk;
    double* w = (double*)malloc(sizeof(double) * (size_t)W);
    if (!w)
        return -1;
    for (long r = row0; r < row1; ++r) {
        const size_t o = (size_t)(r - row0);
        const int h = (int)(r % c->H);
        const float* sg = sigma + o * W;
        const double* gw = dwt + o * W;
        double m = sg[0];
        for (int i = 1; i < W; ++i)
            if (sg[i] > m)
                m = sg[i];
        double z = 0.0;
        for (int i = 0; i < W; ++i)
            z += exp((double)sg[i] - m);
        double mean = 0.0;
        for (int i = 0; i < W; ++i) {
            w[i] = exp((double)sg[i] - m) / z;
            mean += w[i] * gw[i];
        }
        double* gq = dq + o * dk;
        for (int j = 0; j < dk; ++j)
            gq[j] = 0.0;
        for (int i = 0; i < W; ++i) {
            const int32_t n = idx[o * W + i];
            if (n < 0 || n >= S * S) {
                free(w);
                return -1;
            }
            const double ds = w[i] * (gw[i] - mean);
            const int a = n / S, bb = n % S;
            for (int j = 0; j < dh; ++j) {
                const size_t k0 = (((size_t)h * 2 + 0) * S + a) * dh + j;
                const size_t k1 = (((size_t)h * 2 + 1) * S + bb) * dh + j;
                gq[j] += ds * in_value(subkeys, k0, c->in_bf16);
                gq[dh + j] += ds * in_value(subkeys, k1, c->in_bf16);
                dsub[k0] += ds * in_value(q, (size_t)r * dk + j, c->in_bf16);
                dsub[k1] += ds * in_value(q, (size_t)r * dk + dh + j, c->in_bf16);
            }
        }
    }
    free(w);
    return 0;
}
