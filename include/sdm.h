/*
 * sdm.h -- C ABI of the Sparse Delta Memory (SDM) layer forward pass on AMD
 * MI355X (gfx950).
 *
 * The operation (SDM blog post, lcabannes.github.io/sdm-blogpost, section
 * "How does SDM work?", its "Write & Read" subsection and the caption of the
 * figure "The SDM mechanism, end to end"): each (sequence b, head h) owns a
 * memory of N = S*S slot vectors of width d.  For every token t, in order:
 *   1. addressing: the write query wq[b,t,h] is split into two halves; half 0
 *      is scored against sub-key table 0 and half 1 against table 1 (S
 *      sub-keys each); each half keeps its k best sub-keys; every pair (a, b)
 *      of survivors is a candidate slot n = a*S + b scored by the float sum of
 *      its two half scores; the W best candidates are selected and weighted by
 *      a softmax of their sums.  The read query rq[b,t,h] selects W read slots
 *      with weights the same way, against the same sub-key tables.
 *   2. write: the W write slots are decayed by alpha[b,t,h]; the memory's
 *      prediction vhat = sum_i w_i x_i of v[b,t,h] is formed from the decayed
 *      slots x_i; each slot becomes x_i + w_i * beta[b,t,h] * (v - vhat).
 *   3. read: out[b,t,h] = sum_j r_j * M[m_j], after the write of the same token.
 * Orders are by score descending, then index ascending.  Slots that are not
 * written keep their value.  All arithmetic is float32; a bf16 state is
 * rounded to nearest-even when a slot is stored.
 *
 * Layouts (row-major, innermost last; all pointers are DEVICE pointers owned
 * by the caller, 16-byte aligned):
 *   wq, rq    [B, T, H, dk]    in_dtype
 *   v         [B, T, H, d]     in_dtype
 *   alpha     [B, T, H]        float32, the decay of the write-selected slots
 *   beta      [B, T, H]        float32, the delta-rule step size
 *   subkeys   [H, 2, S, dk/2]  in_dtype, table 0 then table 1 per head
 *   mem_inout [B, H, N, d]     state_dtype, slot-major: slot n's d values are
 *                              contiguous; read as the initial memory and
 *                              overwritten with the memory after token T-1.
 *                              Consecutive slot rows are mem_stride elements
 *                              apart (sdm_config; d when it is 0): the tensor
 *                              is [B, H, N, mem_stride] with elements d and up
 *                              of each row never read or written
 *   out       [B, T, H, d]     float32
 *   idx, wt   [B*T*H, W]       int32 slot ids / float32 weights, best first
 *   scores    [B*T*H, 2, S]    float32 half scores
 *
 * Errors: every entry point returns a status and never throws.  Arguments are
 * checked on the host before anything is launched; on any error nothing is
 * launched and sdm_last_error() describes it.  NaN/Inf inputs are not checked
 * and propagate.  Calls are asynchronous on the stream given to sdm_create;
 * the library never synchronises the stream except in sdm_get_timing.
 * A handle must not be used from two host threads at once.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDM_ABI_VERSION 2

#if defined(__GNUC__)
#define SDM_API __attribute__((visibility("default")))
#else
#define SDM_API
#endif

typedef struct sdm_ctx* sdm_handle;

typedef enum {
    SDM_OK = 0,
    SDM_ERR_INVALID_ARG = 1, /* a null/misaligned pointer, a bad handle, an inconsistent shape */
    SDM_ERR_UNSUPPORTED = 2, /* a valid shape outside what the kernels implement */
    SDM_ERR_OOM = 3,         /* device workspace allocation failed */
    SDM_ERR_DEVICE = 4       /* a HIP runtime error */
} sdm_status;

typedef enum { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

typedef struct {
    int B;      /* sequences */
    int H;      /* heads: independent memories and sub-key tables per sequence */
    int T;      /* tokens per call */
    int d;      /* slot width */
    int n_sub;  /* S, sub-keys per table; N = S*S slots */
    int dk;     /* query width; each half is dk/2 */
    int k;      /* per-half candidates */
    int W;      /* slots selected per token, for the write and for the read */
    sdm_dtype in_dtype;    /* wq, rq, v, subkeys */
    sdm_dtype state_dtype; /* mem_inout */
    int mem_stride;        /* elements from one slot row to the next in every state tensor
                              (mem_inout; dmem_inout of sdm_backward, in float32 elements; m0 and
                              mem_out of sdm_broadcast_memory): 0 for dense rows (d), else at least
                              d with mem_stride * sizeof(state) a multiple of 16 bytes; see
                              sdm_mem_stride_hint */
} sdm_config;

/* Accumulated device time per kernel (milliseconds) since timing was enabled. */
typedef struct {
    double ms_score;   /* sub-key scoring (MFMA) */
    double ms_select;  /* per-half top-k, top-W, softmax */
    double ms_plan;    /* the scan's plan: packed slot records, forwarding and store decisions */
    double ms_scan;    /* the memory scan */
    long long n_score, n_select, n_plan, n_scan; /* launches timed */
    double ms_step;    /* decode steps (sdm_step), both of their kernels */
    long long n_step;  /* steps timed */
    double ms_train;     /* the logging scan of sdm_forward_train */
    double ms_bwd_scan;  /* the reverse walk of sdm_backward */
    double ms_bwd_rows;  /* per-row work: conflict flags, reduction, softmax derivative, query gradients */
    double ms_bwd_sub;   /* sub-key gradients */
    long long n_train, n_bwd_scan, n_bwd_rows, n_bwd_sub;
    double ms_project;   /* input projections (sdm_project) */
    long long n_project;
} sdm_timing;

/* Supported shapes: 1 <= k <= min(S, 64); 1 <= W <= min(k*k, 64); S <= 1024;
 * dk/2 a multiple of 16 and at most 256; d a multiple of 8;
 * N*mem_stride*sizeof(state) below 2^32 bytes per memory. */

/* A slot-row stride (elements, for sdm_config.mem_stride) that the scans run
 * faster on: a dense row of 2m 128-byte units padded to 2m + 1 (d itself when
 * the row is an odd number of units, is not a multiple of 128 bytes or is
 * under 1 KB).  The scan reads and writes one 128-byte segment of each selected
 * row per workgroup; with rows a multiple of 256 bytes apart the same segment
 * of every row falls on a subset of the memory channels.  Measured on MI355X
 * with the scan's access pattern (random rows, two segments read per segment
 * written): 8192-byte rows 4.5 TB/s dense, 5.1 TB/s 8320 bytes apart.  The
 * padding costs (stride - d) / d more memory.  Returns 0 for a NULL cfg. */
SDM_API int sdm_mem_stride_hint(const sdm_config* cfg);

/* Validate cfg, allocate the device workspace and bind the HIP stream
 * (a hipStream_t, NULL for the default stream).  *out receives the handle.
 * The device is the one current on the calling thread. */
SDM_API sdm_status sdm_create(const sdm_config* cfg, void* hip_stream, sdm_handle* out);

/* The whole layer forward for B sequences of T tokens: addressing of wq and rq,
 * then the scan.  mem_inout is updated in place; out receives the reads. */
SDM_API sdm_status sdm_forward(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* mem_inout, float* out);

/* One token of the layer over a persistent memory (decode): the same operation
 * as sdm_forward with T = 1 for B sequences and H heads, in one or two launches
 * sized for a single token; T consecutive steps leave exactly the memory and outputs
 * of one T-token forward.  Tensors of the token: wq, rq [B, H, dk] in_dtype;
 * v [B, H, d] in_dtype; alpha, beta [B, H] float32; out [B, H, d] float32;
 * subkeys and mem_inout as for sdm_forward.  The handle's T is not used.
 * SDM_ERR_UNSUPPORTED unless d * sizeof(state) is a multiple of 128 bytes.
 * (SDM blog post, section "How does SDM work?": the per-token update whose
 * cost does not grow with the sequence.) */
SDM_API sdm_status sdm_step(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                            const float* beta, const void* subkeys, void* mem_inout, float* out);

/* sdm_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * handle, no allocation and no library routine that allocates.  cfg, the
 * stream (a hipStream_t, NULL for the default stream) and the token's tensors
 * as for sdm_step on a handle made from cfg (cfg->T is not used); the result
 * equals sdm_step's bit for bit.  Where sdm_step runs two launches (float32
 * queries, or a shape outside its one-launch form) the slot ids and weights
 * pass between them through a 1 MiB array in device memory that the library
 * holds on each device until the process ends, so B*H*W may be at most 65536
 * (SDM_ERR_UNSUPPORTED beyond; nothing launched).  The array holds no state
 * between calls (every entry a call reads, the same call writes first), but
 * calls that overlap on one device share it and race: issue them in order, on
 * one stream or with events between streams.  Other errors as for sdm_step. */
SDM_API sdm_status sdm_step_static(const sdm_config* cfg, void* hip_stream, const void* wq, const void* rq,
                                   const void* v, const float* alpha, const float* beta, const void* subkeys,
                                   void* mem_inout, float* out);

/* Training forward: exactly sdm_forward's memory and outputs (the same
 * launches; the scan also stores), and the bits of every write slot before its
 * write, saved to log [B, H, T, W, d] (state dtype, dense rows; entry
 * ((b*H + h)*T + t)*W + i is write position i of token t, best first), which
 * sdm_backward consumes.  The log holds B*H*T*W*d*sizeof(state) bytes (17.2 GB
 * for B=4, H=1, T=8192, W=64, d=2048, float32), owned by the caller.
 * SDM_ERR_UNSUPPORTED unless d * sizeof(state) is a multiple of 128 bytes and
 * one memory's log of a scan chunk (up to 3072 tokens) stays below 4 GiB.  (SDM blog post, section "How does SDM
 * work?": the decay and delta-rule write whose inputs the log keeps.) */
SDM_API sdm_status sdm_forward_train(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                                     const float* beta, const void* subkeys, void* mem_inout, float* out, void* log);

/* Device bytes sdm_backward allocates on its first call on a handle (kept
 * until sdm_destroy): per-column partial sums [B*T*H, d/32, 2W+2], dense
 * softmax-derivative rows [2, B*T*H, 2, S] and split sub-key sums, all float32,
 * one flag per row and an 8 KB sink. */
SDM_API sdm_status sdm_backward_workspace_bytes(const sdm_config* cfg, size_t* bytes);

/* Backward pass of sdm_forward_train, by reverse-mode differentiation of the
 * forward (SDM blog post, section "How does SDM work?", its "Write & Read"
 * subsection and the caption of the figure "The SDM mechanism, end to end"):
 * the selected slots are held fixed (top-k and top-W are piecewise constant),
 * and the rounding of stored values is passed straight through.
 * Inputs as given to sdm_forward_train (wq, rq, v, alpha, beta, subkeys), and:
 *   mem_inout  state [B, H, N, d]: the memory sdm_forward_train left; the
 *              reverse walk restores it, bit for bit, to the memory before it
 *   log        that call's log [B, H, T, W, d], read only
 *   dout       float32 [B, T, H, d]: dL/d(out)
 *   dmem_inout float32 [B, H, N, d], rows mem_stride float32 elements apart:
 *              in dL/d(final memory) (zeros if the loss does not use it),
 *              out dL/d(initial memory)
 * Outputs, float32, overwritten: dwq, drq [B, T, H, dk]; dv [B, T, H, d];
 * dalpha, dbeta [B, T, H]; dsubkeys [H, 2, S, dk/2].
 * The addressing of both query sets is recomputed by the forward's kernels, so
 * the slots are those the forward used.  Allocates its workspace on the first
 * call (sdm_backward_workspace_bytes).  Deterministic: every sum has a fixed
 * order.  SDM_ERR_UNSUPPORTED for the shapes sdm_forward_train rejects. */
SDM_API sdm_status sdm_backward(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                                const float* beta, const void* subkeys, void* mem_inout, const void* log,
                                const float* dout, float* dmem_inout, float* dwq, float* drq, float* dv,
                                float* dalpha, float* dbeta, float* dsubkeys);

/* The layer's input projections for the call's B*T tokens (SDM blog post,
 * section "How does SDM work?", its "Write & Read" subsection: the token
 * embedding projected to the write keys and, separately, to the read query;
 * the value and the gates of the gated delta rule from the same embedding).
 * Per token and head, with C = 2*dk + d + 2 output rows per head:
 *   wq = x Wq^T, rq = x Wr^T, v = x Wv^T               (bf16, nearest even)
 *   alpha = sigmoid(x wa + bias[h][0]), beta = sigmoid(x wb + bias[h][1])  (float32)
 *   x         [B, T, D] bf16 (D a multiple of 8), the embedding
 *   w         [H*C, D] bf16: head h's rows h*C + [0,dk) Wq, [dk,2dk) Wr,
 *             [2dk, 2dk+d) Wv, 2dk+d wa, 2dk+d+1 wb (an output's D weights contiguous)
 *   gate_bias [H, 2] float32
 *   wq, rq    [B, T, H, dk] bf16; v [B, T, H, d] bf16; alpha, beta [B, T, H] float32:
 *             exactly the inputs sdm_forward takes.
 * One MFMA launch; float32 accumulation, one rounding per output.
 * SDM_ERR_UNSUPPORTED unless in_dtype is bf16. */
SDM_API sdm_status sdm_project(sdm_handle h, int D, const void* x, const void* w, const float* gate_bias, void* wq,
                               void* rq, void* v, float* alpha, float* beta);

/* A learned initial memory m0 [H, N, d] (state dtype) copied into each of the
 * B sequences' memories mem_out [B, H, N, d], ready for sdm_forward.  Both
 * have rows mem_stride elements apart; the copy includes the padding. */
SDM_API sdm_status sdm_broadcast_memory(sdm_handle h, const void* m0, void* mem_out);

/* Diagnostic, not part of the layer: the write/read bucket overlap of the SDM
 * blog post's needle-in-a-haystack figure (section "Memory Access Patterns on
 * a Needle-in-a-Haystack Task"), from a call's addressing idx_w, wt_w, idx_r,
 * wt_r [B*T*H, W] (as sdm_address gives them; row (b*T + t)*H + h).  Slot n
 * falls in bucket n * buckets / N (a contiguous slot range; buckets = S gives
 * the first sub-key).  Outputs, float32, overwritten:
 *   write_cum [B, H, T, buckets]  write weight landed in each bucket by tokens 0..t
 *   read      [B, H, T, buckets]  token t's read weight in each bucket
 *   overlap   [B, H, n_queries, T]  for query token q = queries[i] (device
 *             int32 array) and token a <= q: the sum over the slots token a
 *             writes and token q reads of w_a * r_q; 0 for a > q and for a
 *             query outside [0, T).
 * Sums in double, each value rounded once. */
SDM_API sdm_status sdm_overlap(sdm_handle h, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                               const float* wt_r, int buckets, float* write_cum, float* read, int n_queries,
                               const int32_t* queries, float* overlap);

/* Free the workspace and the handle.  Waits for the handle's stream first. */
SDM_API sdm_status sdm_destroy(sdm_handle h);

/* Static text for a status code. */
SDM_API const char* sdm_status_str(sdm_status s);

/* Text of the last error on the calling host thread ("" if none). */
SDM_API const char* sdm_last_error(void);

/* Device workspace bytes sdm_create would allocate for cfg. */
SDM_API sdm_status sdm_workspace_bytes(const sdm_config* cfg, size_t* bytes);

/* Stage seams (the same kernels sdm_forward runs), for staged checking.
 * sdm_score:     half scores of the B*T*H rows of q            -> scores
 * sdm_select:    top-k / outer-sum top-W / softmax of scores   -> idx, wt
 * sdm_address:   the forward's addressing of the B*T*H rows of q -> idx, wt
 *                (scores kept internal; the scores that can reach a half's
 *                top k recomputed exactly, as sdm_forward does) 
 * sdm_address_pair: both query sets at once, as sdm_forward launches them
 *                (one scoring and one selection launch for wq and rq)
 *                -> idx_w, wt_w and idx_r, wt_r; the same values as two
 *                sdm_address calls
 * sdm_scan_with: the scan driven by given write and read addressing */
SDM_API sdm_status sdm_score(sdm_handle h, const void* q, const void* subkeys, float* scores);
SDM_API sdm_status sdm_select(sdm_handle h, const float* scores, int32_t* idx, float* wt);
SDM_API sdm_status sdm_address(sdm_handle h, const void* q, const void* subkeys, int32_t* idx, float* wt);
SDM_API sdm_status sdm_address_pair(sdm_handle h, const void* wq, const void* rq, const void* subkeys,
                                    int32_t* idx_w, float* wt_w, int32_t* idx_r, float* wt_r);
SDM_API sdm_status sdm_scan_with(sdm_handle h, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                         const float* wt_r, const void* v, const float* alpha, const float* beta,
                         void* mem_inout, float* out);

/* Per-kernel timing with HIP events recorded on the handle's stream around
 * every launch.  sdm_get_timing waits for the recorded events, adds them to the
 * totals and returns the totals; enabling again resets them. */
SDM_API sdm_status sdm_set_timing(sdm_handle h, int enable);
SDM_API sdm_status sdm_get_timing(sdm_handle h, sdm_timing* t);

/* Measurement, not part of the layer: the memory traffic of the scan with its
 * arithmetic taken out.  For each of `memories` memories of `rows` rows of
 * row_bytes bytes (device pointer mem, 16-byte aligned, row_bytes a multiple of
 * 128, one memory below 4 GiB) and each of T tokens: W rows read as the write
 * set, W rows read as the read set and the W write rows stored, each as one
 * 128-byte segment per workgroup, on rows drawn by a hash of (seed, memory,
 * token, set, position).  3*W*row_bytes*T*memories bytes move per call; the
 * contents of mem are scrambled.  Asynchronous on hip_stream (a hipStream_t).
 * The bandwidth it reaches is what random 128-byte reads and writes in the
 * scan's 2:1 mix allow on the device, the ceiling of the scan's access pattern. */
SDM_API sdm_status sdm_pattern_probe(void* mem, int memories, long rows, int row_bytes, int T, int W,
                                     unsigned seed, void* hip_stream);

/* The same with `reads` row segments read and the first `writes` of them stored
 * back per slot position and token: 2:1 is sdm_pattern_probe; 4:3 is the
 * reverse scan of sdm_backward (the read slot's memory and gradient, the write
 * slot's gradient and logged value read; both gradients and the restored
 * memory written), the ceiling of its access pattern.  Rows are row_stride
 * bytes apart (0: row_bytes; else at least row_bytes, a multiple of 16), as a
 * padded memory's are.  (reads + writes) * W * row_bytes * T * memories bytes
 * move per call.  Other mixes: SDM_ERR_INVALID_ARG. */
SDM_API sdm_status sdm_pattern_probe_mix(void* mem, int memories, long rows, int row_bytes, long row_stride, int T,
                                         int W, int reads, int writes, unsigned seed, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SDM_H */
