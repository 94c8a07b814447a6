/*
 * Reference oracle for the SDM layer's input projections.
 *
 * TEST INFRASTRUCTURE, like sdm_oracle.h: only the test-suite and the smoke
 * check may load this library; the GPU library never links or calls it.
 *
 * The SDM blog post (section "How does SDM work?", its "Write & Read"
 * subsection) projects the token embedding to the write keys and, separately,
 * to the query that selects the read slots; the layer extends Gated DeltaNet,
 * whose value and gates are projections of the same embedding.  Readings (the
 * pages give no formula): per head, linear projections without bias for the
 * write query, the read query and the value; the decay and the step size are
 * sigmoids of a linear projection plus a bias; every head sees the whole
 * embedding.
 *
 * Layouts (row-major, innermost last; row r = b*T + t):
 *   x       [B, T, D]          bf16 bits
 *   w       [H * C, D]         bf16 bits, C = 2*dk + d + 2: for head h the rows
 *                              h*C + [0, dk) give wq, [dk, 2dk) rq, [2dk, 2dk+d) v,
 *                              2dk+d alpha's logit, 2dk+d+1 beta's logit
 *                              (each output's D weights contiguous)
 *   bias    [H, 2]             float32: alpha's and beta's bias
 *   wq, rq  [B, T, H, dk]      bf16 bits (nearest-even from the exact sum)
 *   v       [B, T, H, d]       bf16 bits
 *   alpha, beta [B, T, H]      float32: sigmoid(sum + bias), in double, rounded once
 * Sums are accumulated in double.  Returns 0, or -1 on a rejected argument.
 */
#ifndef SDM_ORACLE_PROJ_H
#define SDM_ORACLE_PROJ_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oracle_project(int B, int T, int H, int D, int dk, int d, const uint16_t* x, const uint16_t* w,
                   const float* bias, long row0, long row1, uint16_t* wq, uint16_t* rq, uint16_t* v, float* alpha,
                   float* beta);

/* The initial memory m0 [H, N, d] (n_bytes_each = N*d*elem bytes per head)
 * copied into each of the B sequences' memories mem [B, H, N, d]. */
int oracle_broadcast_memory(int B, int H, long bytes_per_head, const void* m0, void* mem);

#ifdef __cplusplus
}
#endif
#endif
