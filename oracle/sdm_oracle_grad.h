/*
 * Reference oracle for the gradient (backward pass) of the Sparse Delta Memory
 * (SDM) layer.
 *
 * TEST INFRASTRUCTURE, like sdm_oracle.h: only the test-suite may load this
 * library.  It is built from this file's source together with sdm_oracle.c,
 * whose forward it replays; the GPU library never links or calls either.
 *
 * What is differentiated is the forward of sdm_oracle.h (SDM blog post,
 * section "How does SDM work?", its "Write & Read" subsection and the caption
 * of the figure "The SDM mechanism, end to end").  Reverse-mode
 * differentiation of it, with two readings the pages leave open:
 *   - the selected slots are constants: top-k and top-W are piecewise constant
 *     in the queries, so gradients reach the queries and sub-keys only through
 *     the softmax weights of the slots that were selected;
 *   - the rounding of a stored value to the state type is the identity for
 *     the gradient (straight-through).
 * Gradients are computed in double.
 *
 * Layouts are those of sdm_oracle.h; every gradient array has the layout of
 * the value it is the gradient of, in double.
 */
#ifndef SDM_ORACLE_GRAD_H
#define SDM_ORACLE_GRAD_H
#include "sdm_oracle.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Gradient of the scan of memory (b, h) over all T tokens and d elements.
 * mem0      [B,H,N,d]  the memory before the forward, in c->state_bf16's storage
 * dout      [B,T,H,d]  float32, dL/d(out)
 * dmem      [B,H,N,d]  double; in: dL/d(final memory), out: dL/d(mem0) (memory (b, h) only)
 * dv        [B,T,H,d]  double, written for the rows of (b, h)
 * dalpha, dbeta [B,T,H] double, written for the rows of (b, h)
 * dwt_w, dwt_r  [B*T*H, W] double: dL/d(write weights), dL/d(read weights)
 * The forward is replayed from mem0 to record the value of every write slot
 * before its write; the reverse walk then restores those values token by
 * token, so each read sees the memory it saw in the forward. */
int oracle_scan_grad(const oracle_cfg* c, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                     const float* wt_r, const void* v, const float* alpha, const float* beta, const void* mem0,
                     const float* dout, double* dmem, double* dv, double* dalpha, double* dbeta, double* dwt_w,
                     double* dwt_r, int b, int h);

/* Weights of W given slots for one query, in double throughout (no rounding
 * of scores or sums): sigma_i = <q[0:dh], K0[a_i]> + <q[dh:dk], K1[b_i]> with
 * slot n_i = a_i*S + b_i, then w = softmax(sigma).  q [dk] and subkeys
 * [H,2,S,dh] are double; h is the query's head.  For derivative checks. */
int oracle_weights_f64(const oracle_cfg* c, const double* q, const double* subkeys, int h, const int32_t* slot,
                       double* w);

/* Gradient of addressing rows [row0, row1) through the softmax weights of the
 * selected slots.  idx, sigma [rows, W]: the forward's slots and float sums
 * (oracle_address); dwt [rows, W] double: dL/d(weights).
 * dq [rows, dk] double is written; dsub [H,2,S,dh] double is accumulated. */
int oracle_address_grad(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                        const int32_t* idx, const float* sigma, const double* dwt, double* dq, double* dsub);

#ifdef __cplusplus
}
#endif
#endif
