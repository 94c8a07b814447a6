/*
 * Reference oracle for the SDM layer's input projections.
 * TEST INFRASTRUCTURE: see sdm_oracle_proj.h for who may use it, the layouts
 * and the readings taken.  Plain and sequential.
 */
#include "sdm_oracle_proj.h"

#include <math.h>
#include <string.h>

uint16_t oracle_bf16_round(double x); /* sdm_oracle.c */

static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* One output of one row: the dot product of the row's embedding with the
 * output's weight row, in double. */
static double dot(const uint16_t* xr, const uint16_t* wr, int D)
{
    double s = 0.0;
    for (int k = 0; k < D; ++k)
        s += bf(xr[k]) * bf(wr[k]);
    return s;
}

int oracle_project(int B, int T, int H, int D, int dk, int d, const uint16_t* x, const uint16_t* w,
                   const float* bias, long row0, long row1, uint16_t* wq, uint16_t* rq, uint16_t* v, float* alpha,
                   float* beta)
{
    if (B < 1 || T < 1 || H < 1 || D < 1 || dk < 1 || d < 1 || !x || !w || !bias || !wq || !rq || !v || !alpha ||
        !beta || row0 < 0 || row1 > (long)B * T || row0 > row1)
        return -1;
    const long C = 2L * dk + d + 2;
    for (long r = row0; r < row1; ++r) {
        const uint16_t* xr = x + r * D;
        for (int h = 0; h < H; ++h) {
            const uint16_t* wh = w + (size_t)h * C * D;
            const size_t o = (size_t)r * H + h; /* (b, t, h) */
            for (int j = 0; j < dk; ++j) {
                wq[o * dk + j] = oracle_bf16_round(dot(xr, wh + (size_t)j * D, D));
                rq[o * dk + j] = oracle_bf16_round(dot(xr, wh + (size_t)(dk + j) * D, D));
            }
            for (int j = 0; j < d; ++j)
                v[o * d + j] = oracle_bf16_round(dot(xr, wh + (size_t)(2 * dk + j) * D, D));
            const double za = dot(xr, wh + (size_t)(2 * dk + d) * D, D) + bias[2 * h];
            const double zb = dot(xr, wh + (size_t)(2 * dk + d + 1) * D, D) + bias[2 * h + 1];
            alpha[o] = (float)(1.0 / (1.0 + exp(-za)));
            beta[o] = (float)(1.0 / (1.0 + exp(-zb)));
        }
    }
    return 0;
}

int oracle_broadcast_memory(int B, int H, long bytes_per_head, const void* m0, void* mem)
{
    if (B < 1 || H < 1 || bytes_per_head < 1 || !m0 || !mem)
        return -1;
    for (int b = 0; b < B; ++b)
        memcpy((char*)mem + (size_t)b * H * bytes_per_head, m0, (size_t)H * bytes_per_head);
    return 0;
}
