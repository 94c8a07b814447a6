/*
 * Reference oracle for the Sparse Delta Memory (SDM) layer forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What is computed follows the SDM blog post (lcabannes.github.io/sdm-blogpost),
 * section "How does SDM work?", its "Write & Read" subsection and the caption
 * of the figure "The SDM mechanism, end to end":
 *   - a memory of N slot vectors of width d per (sequence, head);
 *   - product-key addressing: two sub-key score sets, per-half top-k, the
 *     outer sum of the two candidate lists, top-W of those sums;
 *   - a gated delta-rule write to the W write-selected slots (decay first,
 *     then the delta step);
 *   - a softmax-weighted read of the W read-selected slots, after the write.
 * Where the pages leave a step open, the reading taken is stated at the
 * function that takes it.
 *
 * Precision: scores accumulate in double and round once to float; the scan
 * runs in double and rounds once (nearest-even) to the state storage type when
 * a slot is stored; reads see the stored values.
 *
 * Layouts (row-major, innermost last; "row" r = (b*T + t)*H + h):
 *   q        [B,T,H,dk]     float32 or bf16 bits
 *   subkeys  [H,2,S,dk/2]   float32 or bf16 bits
 *   v        [B,T,H,d]      float32 or bf16 bits
 *   alpha    [B,T,H]        float32
 *   beta     [B,T,H]        float32
 *   mem      [B,H,N,d]      float32 or bf16 bits, N = S*S, slot n = a*S + b
 *   idx, wt, sigma [B*T*H, W]  int32 / float32 / float32, best first
 *   scores   [B*T*H, 2, S]  float32
 *   out      [B,T,H,d]      float32
 *
 * Every function returns 0 on success and -1 on an argument it rejects.
 */
#ifndef SDM_ORACLE_H
#define SDM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int B, H, T, d, S, dk, k, W;
    int in_bf16;    /* q, v, subkeys are bf16 bits when 1, float32 when 0 */
    int state_bf16; /* mem is bf16 bits when 1, float32 when 0, float64 when 2 (finite-difference checks) */
} oracle_cfg;

/* bf16 bits nearest (ties to even) to a double; NaN -> quiet NaN. */
uint16_t oracle_bf16_round(double x);

/* Sub-key scores of rows [row0, row1). */
int oracle_scores(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                  float* scores);

/* Indices of the k largest of s[0..n) by (value desc, index asc), best first. */
int oracle_topk(const float* s, int n, int k, int32_t* idx);

/* Outer-sum top-W from the two half score vectors of one row. */
int oracle_select(const float* s1, const float* s2, int S, int k, int W, int32_t* slot, float* sigma);

/* Softmax of W selected sums, in double, rounded to float. */
int oracle_softmax(const float* sigma, int W, float* w);

/* Full addressing (scores -> selection -> weights) for rows [row0, row1). */
int oracle_address(const oracle_cfg* c, const void* q, const void* subkeys, long row0, long row1,
                   int32_t* idx, float* wt, float* sigma);

/* Selection and weights from given scores [rows,2,S] for rows [row0, row1). */
int oracle_address_from_scores(const oracle_cfg* c, const float* scores, long row0, long row1,
                               int32_t* idx, float* wt, float* sigma);

/* Sequential scan over t = 0..T-1 of memory (b, h), for slot elements [e0, e1).
 * mem is read as the initial state and overwritten with the final state. */
int oracle_scan(const oracle_cfg* c, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                const float* wt_r, const void* v, const float* alpha, const float* beta, void* mem,
                float* out, int b, int h, int e0, int e1);

#ifdef __cplusplus
}
#endif
#endif
