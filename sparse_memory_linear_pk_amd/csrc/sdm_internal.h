// Internal declarations shared by the gfx950 kernels and the host API of libsdm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, nearest with ties to even; NaN stays a (quiet) NaN,
// values past the largest finite bfloat16 round to infinity.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return bf16_rne(lo) | (bf16_rne(hi) << 16); }

// order-preserving map from float to uint32 (larger float -> larger key); -0
// and +0 compare equal as floats and get the same key (that of +0)
__device__ __forceinline__ uint32_t ordered_key(float f)
{
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// buffer resources: raw (byte-addressed) buffers; an access past num_records
// reads zeros and drops writes instead of faulting.
// ---------------------------------------------------------------------------

constexpr int kBufferWord3 = 0x00020000; // gfx9-family raw buffer format word

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// ---------------------------------------------------------------------------
// launchers (all asynchronous on `stream`; they return the launch status)
// ---------------------------------------------------------------------------

// Rows of a call.  The per-token tensors are [B, Ts, H, ...]; a launch covers the
// Tc tokens t0 .. t0 + Tc - 1 of every sequence (a chunk of the call, or all of
// it with Tc = Ts, t0 = 0).  Row (b, t, h) is (b * Ts + t) * H + h.
struct Rows {
    int B, H, Tc, Ts, t0;
    __host__ __device__ long count() const { return (long)B * Tc * H; }
};

// Sub-key tables [H, 2, S, dh] (bf16) rearranged into MFMA operand order in
// frag (pk_score_frag_bytes); pk_score's bf16 path reads them from there.
size_t pk_score_frag_bytes(int H, int S, int dh);
hipError_t launch_pk_subkey_frag(const void* subkeys, void* frag, int H, int S, int dh, hipStream_t stream);

// Half scores of the rows of q ([B, Ts, H, dk]) against subkeys [H, 2, S, dh]
// (float32 inputs) or frag (bf16 inputs): scores [B*Ts*H, 2, S], only the
// covered rows written, float32, or binary16 (half_out, bf16 inputs only: the
// forward's candidates for the exact selection).
hipError_t launch_pk_score(const void* q, const void* subkeys, const void* frag, void* scores, const Rows& r,
                           int S, int dh, bool in_bf16, bool half_out, hipStream_t stream);

// Both query sets of the forward at once (q0 -> s0, q1 -> s1), scores stored as
// for half_out = in_bf16: one launch for bf16 inputs with S a multiple of 32.
hipError_t launch_pk_score_pair(const void* q0, const void* q1, const void* subkeys, const void* frag, void* s0,
                                void* s1, const Rows& r, int S, int dh, bool in_bf16, hipStream_t stream);

// Scoring fused with the exact selection's candidate search (bf16 inputs; see
// pk_score.hip): per (half, row) a record of cand_record_dwords(S) words, the
// bitmask of the sub-keys whose float32 score reached the record's threshold,
// then the threshold; records [2][B * Ts * H][RW].  kstat: the tables' mean
// rows and spreads (launch_subkey_stats, subkey_stats_floats(H, dh) floats).
__host__ __device__ inline int cand_record_dwords(int S) { return (S / 32 + 1 + 3) & ~3; }
// candidates per half the threshold aims at
__host__ __device__ inline int cand_target(int k) { return (k + 64) / 2; }
bool pk_cand_path(int S, int dh, int k, bool in_bf16);
size_t subkey_stats_floats(int H, int dh);
hipError_t launch_subkey_stats(const void* subkeys, float* kstat, int H, int S, int dh, hipStream_t stream);
// The fused scoring's whole preparation in one launch: frag (as
// launch_pk_subkey_frag), kmax (max |K| in part 0 of each table, the other
// parts zero) and kstat (as launch_subkey_stats).
hipError_t launch_subkey_prepare(const void* subkeys, void* frag, float* kstat, float* kmax, int H, int S, int dh,
                                 hipStream_t stream);
hipError_t launch_pk_score_cand(const void* q0, const void* q1, const void* frag, const float* kstat, void* rec0,
                                void* rec1, int nsets, const Rows& r, int S, int dh, int k, hipStream_t stream);
// The exact selection from candidate records (nsets query sets; q0, q1 the
// queries the records were made from).
hipError_t launch_pk_topk_cand(const void* rec0, const void* rec1, int32_t* idx0, int32_t* idx1, float* wt0,
                               float* wt1, int nsets, const Rows& r, int S, int k, int W, const void* q0,
                               const void* q1, const void* subkeys, const float* kmax, int dh, hipStream_t stream);

// Per-half top-k, outer-sum top-W and softmax weights of the covered rows:
// scores [B*Ts*H, 2, S] -> idx, wt [B*Ts*H, W].  With q ([B, Ts, H, dk]),
// subkeys and kmax (max |K| per table, [H, 2]) the scores that can reach a
// half's top k are recomputed exactly first (double sums in index order, one
// rounding) and the stored scores are binary16 for bf16 inputs, float32
// otherwise; with q null the float32 scores are taken as given.  kmax: the
// partial maxima of launch_subkey_absmax.
hipError_t launch_pk_topk(const void* scores, int32_t* idx, float* wt, const Rows& r, int S, int k, int W,
                          const void* q, const void* subkeys, const float* kmax, int dh, bool in_bf16,
                          hipStream_t stream);
// The exact selection of both query sets in one launch (q0, q1 required).
hipError_t launch_pk_topk_pair(const void* scores0, const void* scores1, int32_t* idx0, int32_t* idx1, float* wt0,
                               float* wt1, const Rows& r, int S, int k, int W, const void* q0, const void* q1,
                               const void* subkeys, const float* kmax, int dh, bool in_bf16, hipStream_t stream);
// Partial maxima of |K| per sub-key table: kmax[(h * 2 + half) * kAbsmaxParts + p]
// is the largest magnitude in the p-th of kAbsmaxParts slices of table (h, half);
// the selection reduces the parts itself (no atomics, nothing to clear first).
constexpr int kAbsmaxParts = 32;
hipError_t launch_subkey_absmax(const void* subkeys, float* kmax, int H, int S, int dh, bool in_bf16,
                                hipStream_t stream);

// Staged scan: constants shared by its plan and its kernel.
// The kernel steps through tokens in pairs; the slot reads of a pair are issued
// two pairs ahead, its plan records four pairs ahead.
namespace staged {
constexpr int kP = 3;               // a store may be in flight with those of the next kP tokens
constexpr int kWindow = 7;          // tokens back a forwarded value may come from
constexpr int kRing = 12;           // tokens of stored values kept for forwarding (> kWindow)
constexpr int kStages = 6;          // tokens of slot reads in flight or in use (three pairs)
constexpr int kRecSlots = 12;       // tokens of plan records parked in LDS
constexpr int kS0 = -8;             // first (virtual) token: the first pair whose records are loaded holds token 0
constexpr int kPos = 64;            // positions per token (the selection width, padded)
constexpr int kRecs = kPos + 1;     // plan entries per token: one record per position, then the header
constexpr int kSlotBits = 21;       // slot id field; the next 10 bits hold a forwarding source
constexpr uint32_t kDepFlag = 1u;   // header bit (out offset bit 0): the token writes a slot the previous one wrote
static_assert(kRing == kRecSlots && kRecSlots % kStages == 0 && kRecSlots % 4 == 0 && kS0 % 2 == 0,
              "slot rings must line up in the unrolled loop");
static_assert(kRing > kWindow, "forwarding window");
static_assert(kRing * kPos + 1 <= 1024, "forwarding source field");
} // namespace staged

// Launch geometry of the scan, chosen once per shape.
struct ScanPlan {
    bool staged;   // staged kernel (128-byte segments) or the register-ring kernel
    int lps;       // lanes sharing one slot chunk (16 bytes each)
    int rw;        // slot positions per lane
    int waves;     // waves per workgroup
    int lookahead; // tokens between a slot read's issue and its use
    int grid;      // workgroups
    int lds;       // dynamic LDS bytes
    int Tp;        // staged: tokens per memory in the plan (T padded with sentinel tokens)
    int seg_bytes; // staged: bytes of a slot row per workgroup, 128, or 64 (bf16 state, too few memories)
};

// ms: elements from one slot row of a memory to the next (>= d).
bool plan_scan(int B, int H, int T, int d, int ms, int W, long N, bool state_bf16, bool in_bf16, ScanPlan* plan);

// The plan of a forward: per (b, h, t, position) a 16-byte record with the write
// and read slot ids, their weights, where a slot written too recently to be read
// from memory is found instead, and whether its store is superseded; plus the
// token's gates.  Register-ring format: [B*H][T][W] records, then [B*H][T]
// (alpha, beta).  Staged format: [B*H][Tp][65]: 64 records (positions past W and
// tokens past T are sentinels that read nothing and store nothing), then a
// header (alpha, beta, byte offset of the token's v row, of its out row).
size_t plan_bytes(const ScanPlan& p, int B, int H, int T, int W);
// idx/wt [B*Ts*H, W] and alpha/beta [B, Ts, H] are read at the covered rows; the
// plan describes the Tc tokens of the chunk, whose v and out rows it names
// relative to token t0.
hipError_t launch_sdm_plan(const ScanPlan& p, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                           const float* wt_r, const float* alpha, const float* beta, void* plan, const Rows& r,
                           int W, int d, long N, bool in_bf16, hipStream_t stream);

// One chunk's scan: T tokens per memory (the chunk length); v and out point at
// token t0 of sequence 0 and advance Ts tokens per sequence.
struct ScanArgs {
    const uint4* plan;  // records (either format)
    const float2* ab;   // register-ring format: [B*H, T] (alpha, beta)
    const void* v;
    void* mem;
    float* out;
    void* log;          // null, or the write slots' values before each write: memory (b, h) at
                        // log + (b*H + h)*Ts*W*d, token t of the chunk at + t*W*d (staged form only)
    int B, T, Ts, H, d, W, Tp;
    int ms;             // state elements from one slot row to the next (>= d): memory (b, h) at mem + (b*H + h)*N*ms
    long N;
};

hipError_t launch_sdm_scan(const ScanArgs& a, const ScanPlan& plan, bool state_bf16, bool in_bf16,
                           hipStream_t stream);
hipError_t launch_sdm_scan_staged(const ScanArgs& a, const ScanPlan& plan, bool state_bf16, bool in_bf16,
                                  hipStream_t stream);

// One token over a persistent memory (sdm_step): tensors [B, H, ...] of the
// token; idx/wt: workspace of 2*B*H*W entries each; slot rows ms elements apart.
// Needs d * sizeof(state) a multiple of 128 bytes.
bool step_supported(int d, bool state_bf16);
hipError_t launch_sdm_step(const void* wq, const void* rq, const void* v, const float* alpha, const float* beta,
                           const void* subkeys, void* mem, float* out, int32_t* idx, float* wt, int B, int H, int d,
                           int ms, int S, int dh, int k, int W, bool in_bf16, bool state_bf16, hipStream_t stream);

// The backward pass (float32 state with d a multiple of 32, or bf16 state with
// d a multiple of 64: 128-byte memory columns; the gradient is float32).
struct GradArgs {
    int B, H, T, d, S, dh, W;
    int ms;                              // elements from one slot row to the next in mem and G (>= d)
    int ncol;                            // 128-byte memory columns per row: d * sizeof(state) / 128
    bool in_bf16, state_bf16;
    void* mem;                           // [B*H, N, ms] state: memory after the forward in, before it out
    float* G;                            // [B*H, N, ms]: dL/d(memory after) in, dL/d(memory before) out
    const void* log;                     // [B*H, T, W, d] state
    const int32_t* idx[2];               // write, read slots [rows, W]
    const float* wt[2];                  // their weights
    const void* q[2];                    // wq, rq [rows, dk]
    const void* v;                       // [rows, d]
    const float* alpha;                  // [rows]
    const float* beta;                   // [rows]
    const void* subkeys;                 // [H, 2, S, dh]
    const float* dout;                   // [rows, d]
    float* dv;                           // [rows, d]
    float* dalpha;                       // [rows]
    float* dbeta;                        // [rows]
    float* dq[2];                        // dwq, drq [rows, dk]
    float* dsub;                         // [H, 2, S, dh]
    float* part;                         // workspace: [rows, d/32, 2W+2]
    float* ds;                           // workspace: [2, rows, 2, S]
    float* sub_part;                     // workspace: [nsplit, H, 2, S, dh]
    int32_t* conflict;                   // workspace: [rows], token shares a slot with the next one
    float* sink;                         // workspace: kGradSinkBytes, where positions past W go when
                                         // the gradient is addressed with 64-bit pointers
    int nsplit;
};
constexpr size_t kGradSinkBytes = 256 * 32; // a workgroup's lanes x 32 gradient bytes
size_t grad_part_floats(int B, int H, int T, int d, int W, bool state_bf16);
int grad_sub_splits(int B, int H, int T, int S, int dh);
hipError_t launch_grad_conflicts(const GradArgs& a, hipStream_t stream);
hipError_t launch_grad_scan(const GradArgs& a, hipStream_t stream);
hipError_t launch_grad_rows(const GradArgs& a, hipStream_t stream);
hipError_t launch_grad_subkeys(const GradArgs& a, hipStream_t stream);

// Input projections y = x w^T (x [R, D], w [H*(2dk+d+2), D], bf16) with the
// epilogue into wq, rq, v (bf16) and sigmoid gates alpha, beta (float32).
hipError_t launch_project(const void* x, const void* w, const float* bias, void* wq, void* rq, void* v, float* alpha,
                          float* beta, int R, int D, int H, int dk, int d, hipStream_t stream);
// mem[b] = m0 for b < B (bytes_all_heads per sequence, a multiple of 16).
hipError_t launch_broadcast(const void* m0, void* mem, size_t bytes_all_heads, int B, hipStream_t stream);

// The write/read bucket-overlap diagnostic of a call's addressing.
hipError_t launch_overlap(const int32_t* idx_w, const float* wt_w, const int32_t* idx_r, const float* wt_r, int K,
                          float* write_cum, float* read, int Q, const int32_t* queries, float* overlap, int B, int T,
                          int H, int W, long N, hipStream_t stream);

// Measurement only: the scan's traffic pattern without arithmetic on `memories`
// memories of `rows` rows of row_bytes (a multiple of 128) bytes, consecutive
// rows row_stride bytes apart; reads:writes segments per slot position and
// token, 2:1 (the forward scan) or 4:3 (the reverse scan of the backward pass).
hipError_t launch_hbm_pattern(void* mem, int memories, long rows, int row_bytes, long row_stride, int T, int W,
                              int reads, int writes, uint32_t seed, hipStream_t stream);

} // namespace sdm
