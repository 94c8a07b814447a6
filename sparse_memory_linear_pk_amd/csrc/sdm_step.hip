// sdm_step: one token of the SDM layer over a persistent memory (decode).
//
// The same operation as sdm_forward with T = 1 (SDM blog post, section "How
// does SDM work?" and the caption of the figure "The SDM mechanism, end to
// end": addressing of the write and read queries, the decay and delta-rule
// write of the W write slots, then the softmax-weighted read).  For bf16
// queries with 128-wide halves (the workload shapes) and a grid of at most one
// workgroup per CU it is one launch, step_fused_kernel: every workgroup of a
// memory forms that memory's addressing itself, then scans its 128 bytes of the
// rows.  Otherwise two launches sized for a single token:
//
//  1. step_address_kernel: one workgroup per (b, h) scores both queries of the
//     token on the matrix cores, with the instruction, operand layout and
//     reduction order of pk_score (so every score is bit-identical to it), and
//     two of its waves select the write and the read slots with the selection
//     of pk_topk (pk_select.h).
//  2. step_scan_kernel: one workgroup per (b, h, 128 bytes of the slot rows)
//     loads the token's W write and W read segments at once, forms the
//     prediction, updates and stores the write slots, and reads; a read slot
//     that the token wrote takes the stored (rounded) updated value.  Lane
//     mapping, sums and arithmetic are those of the staged scan (scan_cell.h),
//     so T steps leave the memory and outputs of one T-token forward, bit for
//     bit.
#include "pk_select.h"
#include "scan_cell.h"

namespace sdm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

// Running maxima of bf16 magnitudes, two per word (finite bf16 magnitudes order
// as unsigned integers).
__device__ __forceinline__ uint32_t absmax_bf16x8(uint32_t m, const bf16x8_t& v)
{
    const uint4 w = __builtin_bit_cast(uint4, v);
    u16x2_t mm = __builtin_bit_cast(u16x2_t, m);
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2_t, w.x & 0x7FFF7FFFu));
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2_t, w.y & 0x7FFF7FFFu));
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2_t, w.z & 0x7FFF7FFFu));
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2_t, w.w & 0x7FFF7FFFu));
    return __builtin_bit_cast(uint32_t, mm);
}

constexpr int kWaves = 4;

struct StepArgs {
    const void* wq;       // [B, H, dk]
    const void* rq;       // [B, H, dk]
    const void* subkeys;  // [H, 2, S, dh]
    int32_t* idx;         // [2][B*H][W]: write then read slots
    float* wt;            // [2][B*H][W]
    int B, H, S, k, W, n_pairs;
};

// Scores of the two queries of (b, h) against both sub-key tables, into
// sc[query][half][S]: rows 0 (write) and 1 (read) of a 32-row MFMA tile whose
// other rows are zero; the 32 columns are sub-keys.  Operands, instruction and
// k-step order are pk_score's, so each score is the same float.  kmax[half]
// receives this lane's share of max |K| of table `half` (every element of a
// table is loaded by one lane of one wave); the caller reduces over the lanes
// and waves.
template <int DH, bool BF16>
__device__ void step_scores(const StepArgs& a, int bh, float* sc, int lane, int wave, float (&kmax)[2])
{
    const int h = bh % a.H, S = a.S;
    const int i = lane & 31, kg = lane >> 5;
    const int ctiles = (S + 31) / 32;
    const int dk = 2 * DH;
    if constexpr (BF16) {
        // The two queries' operands for both halves once, then the sub-key operands of G
        // tiles at a time: one memory round trip per G tiles instead of per tile.  Each
        // tile's MFMA sequence is unchanged.
        constexpr int KSTEPS = DH / 16, G = 4;
        bf16x8_t qv[2][KSTEPS];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint16_t* q = static_cast<const uint16_t*>(i == 0 ? a.wq : a.rq) + (long)bh * dk + half * DH + kg * 8;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                qv[half][kk] = i < 2 ? *reinterpret_cast<const bf16x8_t*>(q + kk * 16) : bf16x8_t{};
        }
        const int ntask = 2 * ctiles;
        uint32_t km[2] = {0u, 0u};
        for (int t0 = wave; t0 < ntask; t0 += kWaves * G) {
            bf16x8_t bv[G][KSTEPS];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int task = t0 + g * kWaves;
                const int half = task < ntask ? task / ctiles : 0, ct = task < ntask ? task % ctiles : 0;
                const int s = ct * 32 + i;
                const bool on = task < ntask && s < S;
                const uint16_t* krow = static_cast<const uint16_t*>(a.subkeys) + ((long)h * 2 + half) * S * DH +
                                       (long)(on ? s : 0) * DH + kg * 8;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) // a valid row either way; zeroed where used
                    bv[g][kk] = *reinterpret_cast<const bf16x8_t*>(krow + kk * 16);
                if (on) { // rows past S repeat row 0, which another lane covers
                    uint32_t m = 0u;
#pragma unroll
                    for (int kk = 0; kk < KSTEPS; ++kk)
                        m = absmax_bf16x8(m, bv[g][kk]);
                    km[half] = max(km[half], max(m & 0xFFFFu, m >> 16));
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int task = t0 + g * kWaves;
                if (task >= ntask)
                    break; // wave-uniform
                const int half = task / ctiles, ct = task % ctiles;
                const int s = ct * 32 + i;
                f32x16_t acc = {};
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(half ? qv[1][kk] : qv[0][kk],
                                                                  s < S ? bv[g][kk] : bf16x8_t{}, acc, 0, 0, 0);
                // lane l < 32 holds column l of rows 0 (v = 0) and 1 (v = 1)
                if (kg == 0 && s < S) {
                    sc[(0 * 2 + half) * S + s] = acc[0];
                    sc[(1 * 2 + half) * S + s] = acc[1];
                }
            }
        }
        kmax[0] = __uint_as_float(km[0] << 16);
        kmax[1] = __uint_as_float(km[1] << 16);
        return;
    }
    kmax[0] = kmax[1] = 0.f;
    for (int task = wave; task < 2 * ctiles; task += kWaves) {
        const int half = task / ctiles, ct = task % ctiles;
        const int s = ct * 32 + i;
        f32x16_t acc = {};
        {
            constexpr int KSTEPS = DH / 2;
            const float* q = static_cast<const float*>(i == 0 ? a.wq : a.rq) + (long)bh * dk + half * DH + kg;
            const float* table = static_cast<const float*>(a.subkeys) + ((long)h * 2 + half) * S * DH;
            const float* krow = table + (long)(s < S ? s : 0) * DH + kg;
            const float live = s < S ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const float kv = krow[kk * 2] * live;
                kmax[half] = fmaxf(kmax[half], fabsf(kv));
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(i < 2 ? q[kk * 2] : 0.f, kv, acc, 0, 0, 0);
            }
        }
        // lane l < 32 holds column l of rows 0 (v = 0) and 1 (v = 1)
        if (kg == 0 && s < S) {
            sc[(0 * 2 + half) * S + s] = acc[0];
            sc[(1 * 2 + half) * S + s] = acc[1];
        }
    }
}

// Each wave's max |K| of both tables into s_km[wave][half] (visible after the
// next barrier).
__device__ __forceinline__ void publish_kmax(const float (&km)[2], float (*s_km)[2], int lane, int wave)
{
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float m = km[half];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1)
            m = fmaxf(m, __shfl_xor(m, o));
        if (lane == 0)
            s_km[wave][half] = m;
    }
}

__device__ __forceinline__ float kmax_of(const float (*s_km)[2], int half)
{
    return fmaxf(fmaxf(s_km[0][half], s_km[1][half]), fmaxf(s_km[2][half], s_km[3][half]));
}

// The exact-score inputs of query half `half` of memory bh's table, the query
// staged as doubles in qd (pksel::stage_query).
template <int DH, bool BF16>
__device__ __forceinline__ pksel::Refine step_refine(const StepArgs& a, int bh, const double* qd, int half,
                                                     const float (*s_km)[2], int lane)
{
    const size_t es = BF16 ? 2 : 4;
    const int h = bh % a.H;
    pksel::Refine r{qd + half * DH, static_cast<const char*>(a.subkeys) + (size_t)(h * 2 + half) * a.S * DH * es, DH,
                    0.f};
    r.E = pksel::half_bound(r, kmax_of(s_km, half), lane);
    return r;
}

template <int DH, bool BF16, int J, int R>
__global__ __launch_bounds__(kWaves * 64) void step_address_kernel(StepArgs a)
{
    extern __shared__ float s_sc[]; // [query][half][S]
    __shared__ uint64_t s_buf[2][64];
    __shared__ float s_val[2][2][64];
    __shared__ uint32_t s_sub[2][2][64];
    __shared__ uint16_t s_pairs[pksel::kPairsMax];
    __shared__ float s_km[kWaves][2];
    __shared__ double s_qd[2][2 * DH];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    pksel::fill_pairs(s_pairs, a.k, a.W);
    float km[2];
    step_scores<DH, BF16>(a, bh, s_sc, lane, wave, km);
    publish_kmax(km, s_km, lane, wave);
    __syncthreads();
    if (wave < 2) { // wave 0 selects the write slots, wave 1 the read slots
        const long o = ((long)wave * a.B * a.H + bh) * a.W;
        constexpr int es = BF16 ? 2 : 4;
        pksel::stage_query<BF16>(static_cast<const char*>(wave ? a.rq : a.wq) + (size_t)bh * 2 * DH * es, s_qd[wave],
                                 2 * DH, lane);
        const pksel::Refine r0 = step_refine<DH, BF16>(a, bh, s_qd[wave], 0, s_km, lane);
        const pksel::Refine r1 = step_refine<DH, BF16>(a, bh, s_qd[wave], 1, s_km, lane);
        pksel::select_row_exact<J, R, BF16>(s_sc + wave * 2 * a.S, a.S, a.k, a.W, a.n_pairs, s_pairs, lane,
                                            s_buf[wave], s_val[wave], s_sub[wave], a.idx + o, a.wt + o, r0, r1);
    }
}

struct StepScanArgs {
    const int32_t* idx;  // [2][B*H][W]
    const float* wt;     // [2][B*H][W]
    const float* alpha;  // [B*H]
    const float* beta;   // [B*H]
    const void* v;       // [B*H, d]
    void* mem;           // [B*H, N, ms]
    float* out;          // [B*H, d]
    int B, H, d, W;
    long N;
    int ms;              // elements from one slot row to the next
};

// One token for the workgroup's 128 bytes of the rows of memory bh: lane
// (g, e) of wave w holds the 16 bytes e of write and read positions 16w + g
// and 16w + 8 + g, as in the staged scan.  widx/wwt, ridx/rwt: the token's W
// write and read slots and weights (global memory or LDS).
template <class ST, class VT>
__device__ void step_scan_body(const StepScanArgs& a, int bh, int chunk, const int32_t* widx, const float* wwt,
                               const int32_t* ridx, const float* rwt)
{
    using C = Cell<ST>;
    using CT = typename C::CT;
    constexpr int E = C::E;
    constexpr int SEG = 128 / (int)sizeof(ST);
    constexpr int PART = kWaves * 8 * E;                 // partial sums of one kind, [wave][el][E]
    __shared__ __attribute__((aligned(16))) CT s_red[PART];
    __shared__ __attribute__((aligned(16))) float s_ored[PART];
    __shared__ __attribute__((aligned(16))) uint4 s_upd[64 * 8]; // stored values of the write positions
    __shared__ int32_t s_wslot[64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, el = lane & 7;
    const int W = a.W;
    const uint32_t row_bytes = (uint32_t)a.ms * (uint32_t)sizeof(ST); // slot row to slot row
    const uint32_t lane_off = (uint32_t)chunk * 128u + (uint32_t)el * 16u;
    const __amdgpu_buffer_rsrc_t r_mem =
        make_rsrc(static_cast<const char*>(a.mem) + (size_t)bh * a.N * row_bytes, (uint32_t)a.N * row_bytes);
    const int pos[2] = {wave * 16 + g, wave * 16 + 8 + g};

    int32_t ws[2], rs[2];
    float ww[2], rw[2];
    uint4 wv[2], rv[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bool live = pos[p] < W;
        ws[p] = live ? widx[pos[p]] : -1;
        rs[p] = live ? ridx[pos[p]] : -1;
        ww[p] = live ? wwt[pos[p]] : 0.f;
        rw[p] = live ? rwt[pos[p]] : 0.f;
        wv[p] = ld128(r_mem, live ? (uint32_t)ws[p] * row_bytes + lane_off : kOOB);
        rv[p] = ld128(r_mem, live ? (uint32_t)rs[p] * row_bytes + lane_off : kOOB);
    }
    if (el == 0) {
        s_wslot[pos[0]] = ws[0];
        s_wslot[pos[1]] = ws[1];
    }
    const CT al = a.alpha[bh], be = a.beta[bh];
    const CT w0 = ww[0], w1 = ww[1];

    // the prediction of the decayed write slots
    float m0[E], m1[E];
    C::unpack(wv[0], m0);
    C::unpack(wv[1], m1);
    {
        CT acc[E];
#pragma unroll
        for (int q = 0; q < E; ++q)
            acc[q] = predict2<CT>(al, w0, m0[q], w1, m1[q]);
        reduce_to_part<E, CT>(acc, reinterpret_cast<float4*>(s_red), wave, el, lane);
    }
    // v of this lane's elements
    float vv[E];
    {
        const size_t e0 = (size_t)bh * a.d + (size_t)chunk * SEG + (size_t)el * E;
#pragma unroll
        for (int q = 0; q < E; ++q) {
            if constexpr (sizeof(VT) == 2)
                vv[q] = __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.v)[e0 + q] << 16);
            else
                vv[q] = static_cast<const float*>(a.v)[e0 + q];
        }
    }
    __syncthreads();

    // the update: stored to memory and kept for the read
    {
        CT vh[E];
        sum_waves<E, CT>(reinterpret_cast<const float4*>(s_red), el, vh);
        CT y0[E], y1[E];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const CT dlt = delta<CT>(be, vv[q], vh[q]);
            y0[q] = updated<CT>(al, m0[q], w0, dlt);
            y1[q] = updated<CT>(al, m1[q], w1, dlt);
        }
        const uint4 p0 = C::pack(y0), p1 = C::pack(y1);
        s_upd[pos[0] * 8 + el] = p0;
        s_upd[pos[1] * 8 + el] = p1;
        st128(r_mem, ws[0] >= 0 ? (uint32_t)ws[0] * row_bytes + lane_off : kOOB, p0);
        st128(r_mem, ws[1] >= 0 ? (uint32_t)ws[1] * row_bytes + lane_off : kOOB, p1);
    }
    __syncthreads();

    // the read, after the write: a read slot the token wrote takes its stored value
    {
        float q0[E], q1[E];
        uint4 c[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // the 8 lanes of a group search 8 write positions each
            // branch-free: every entry read, the tests combined bitwise (a short-circuit
            // select of this shape has been compiled wrongly elsewhere)
            int hit = -1;
            const int32_t rsp = rs[p];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = el * 8 + t;
                const int32_t sv = s_wslot[j];
                hit = ((j < W) & (sv == rsp) & (rsp >= 0)) ? j : hit;
            }
#pragma unroll
            for (int m = 1; m < 8; m <<= 1)
                hit = max(hit, __shfl_xor(hit, m));
            c[p] = hit >= 0 ? s_upd[hit * 8 + el] : rv[p];
        }
        C::unpack(c[0], q0);
        C::unpack(c[1], q1);
        float oa[E];
#pragma unroll
        for (int q = 0; q < E; ++q)
            oa[q] = read2(rw[0], q0[q], rw[1], q1[q]);
        reduce_to_part<E, float>(oa, reinterpret_cast<float4*>(s_ored), wave, el, lane);
    }
    __syncthreads();
    if (wave == 0 && g == 0) {
        float o[E];
        sum_waves<E, float>(reinterpret_cast<const float4*>(s_ored), el, o);
        float* dst = a.out + (size_t)bh * a.d + (size_t)chunk * SEG + (size_t)el * E;
#pragma unroll
        for (int q = 0; q < E; ++q)
            dst[q] = o[q];
    }
}

template <class ST, class VT>
__global__ __launch_bounds__(kWaves * 64) void step_scan_kernel(StepScanArgs a)
{
    const int nchunk = a.d / (128 / (int)sizeof(ST));
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const long wrow = (long)bh * a.W, rrow = ((long)a.B * a.H + bh) * a.W;
    step_scan_body<ST, VT>(a, bh, chunk, a.idx + wrow, a.wt + wrow, a.idx + rrow, a.wt + rrow);
}

// The whole step in one launch, for bf16 queries: every workgroup of memory bh
// forms bh's addressing itself (the same scores and selection as
// step_address_kernel, the four half selections on the four waves at once, the
// two top-W selections on two of them), then scans its 128 bytes.  The
// repeated addressing runs in parallel, so it adds no latency.
template <int DH, int J, int R, class ST>
__global__ __launch_bounds__(kWaves * 64) void step_fused_kernel(StepArgs a, StepScanArgs c)
{
    extern __shared__ float s_sc[]; // [query][half][S]
    __shared__ uint64_t s_buf[kWaves][64];
    __shared__ float s_val[2][2][64];
    __shared__ uint32_t s_sub[2][2][64];
    __shared__ uint16_t s_pairs[pksel::kPairsMax];
    __shared__ int32_t s_idx[2][64];
    __shared__ float s_wt[2][64];
    __shared__ float s_km[kWaves][2];
    __shared__ double s_qd[kWaves][2 * DH];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nchunk = c.d / (128 / (int)sizeof(ST));
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    pksel::fill_pairs(s_pairs, a.k, a.W);
    float km[2];
    step_scores<DH, true>(a, bh, s_sc, lane, wave, km);
    publish_kmax(km, s_km, lane, wave);
    __syncthreads();
    {
        const int q = wave >> 1, half = wave & 1; // waves 0, 1: write query; 2, 3: read query
        pksel::stage_query<true>(static_cast<const char*>(q ? a.rq : a.wq) + (size_t)bh * 2 * DH * 2, s_qd[wave],
                                 2 * DH, lane);
        const pksel::Refine ref = step_refine<DH, true>(a, bh, s_qd[wave], half, s_km, lane);
        pksel::select_half_exact<J, true>(s_sc + (q * 2 + half) * a.S, a.S, a.k, lane, s_buf[wave], s_val[q][half],
                                          s_sub[q][half], ref);
    }
    __syncthreads();
    if (wave < 2)
        pksel::select_from_lists<R>(a.S, a.k, a.W, a.n_pairs, s_pairs, lane, s_buf[wave], s_val[wave], s_sub[wave],
                                    s_idx[wave], s_wt[wave]);
    __syncthreads();
    step_scan_body<ST, uint16_t>(c, bh, chunk, s_idx[0], s_wt[0], s_idx[1], s_wt[1]);
}

template <int DH, bool BF16, int J>
hipError_t launch_address_j(const StepArgs& a, hipStream_t stream)
{
    const size_t lds = (size_t)4 * a.S * sizeof(float);
#define SDM_STEP_R(Rv)                                                                                        \
    if (a.n_pairs <= 64 * Rv) {                                                                               \
        hipLaunchKernelGGL((step_address_kernel<DH, BF16, J, Rv>), dim3((unsigned)(a.B * a.H)),             \
                           dim3(kWaves * 64), lds, stream, a);                                                \
        return hipGetLastError();                                                                             \
    }
    SDM_STEP_R(1)
    SDM_STEP_R(2)
    SDM_STEP_R(4)
    SDM_STEP_R(8)
#undef SDM_STEP_R
    return hipErrorInvalidValue;
}

template <int DH, bool BF16>
hipError_t launch_address_dh(const StepArgs& a, hipStream_t stream)
{
    if (a.S <= 64)
        return launch_address_j<DH, BF16, 1>(a, stream);
    if (a.S <= 128)
        return launch_address_j<DH, BF16, 2>(a, stream);
    if (a.S <= 256)
        return launch_address_j<DH, BF16, 4>(a, stream);
    if (a.S <= 512)
        return launch_address_j<DH, BF16, 8>(a, stream);
    return launch_address_j<DH, BF16, 16>(a, stream);
}

template <bool BF16>
hipError_t launch_address(const StepArgs& a, int dh, hipStream_t stream)
{
    switch (dh) {
    case 16: return launch_address_dh<16, BF16>(a, stream);
    case 32: return launch_address_dh<32, BF16>(a, stream);
    case 48: return launch_address_dh<48, BF16>(a, stream);
    case 64: return launch_address_dh<64, BF16>(a, stream);
    case 96: return launch_address_dh<96, BF16>(a, stream);
    case 128: return launch_address_dh<128, BF16>(a, stream);
    case 192: return launch_address_dh<192, BF16>(a, stream);
    case 256: return launch_address_dh<256, BF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

bool step_supported(int d, bool state_bf16) { return (d * (state_bf16 ? 2 : 4)) % 128 == 0; }

hipError_t launch_sdm_step(const void* wq, const void* rq, const void* v, const float* alpha, const float* beta,
                           const void* subkeys, void* mem, float* out, int32_t* idx, float* wt, int B, int H, int d,
                           int ms, int S, int dh, int k, int W, bool in_bf16, bool state_bf16, hipStream_t stream)
{
    if (!step_supported(d, state_bf16) || S > 1024 || k > 64 || W > 64 || ms < d ||
        (uint64_t)S * S * ms * (state_bf16 ? 2 : 4) >= (1ull << 32))
        return hipErrorInvalidValue;
    StepArgs sa{wq, rq, subkeys, idx, wt, B, H, S, k, W, pksel::pair_count(k, W)};
    if (sa.n_pairs > pksel::kPairsMax)
        return hipErrorInvalidValue;
    StepScanArgs ca{idx, wt, alpha, beta, v, mem, out, B, H, d, W, (long)S * S, ms};
    const int nchunk = d * (state_bf16 ? 2 : 4) / 128;
    dim3 grid((unsigned)(B * H * nchunk)), block(kWaves * 64);
    // one launch for the workload shapes (bf16 queries, 128-wide halves) when
    // every workgroup has a CU of its own (more would repeat the addressing on
    // shared CUs, which costs more than the second launch saves)
    if (in_bf16 && dh == 128 && S > 256 && sa.n_pairs <= 256 && B * H * nchunk <= 256) {
        const size_t lds = (size_t)4 * S * sizeof(float);
        if (S <= 512)
            hipLaunchKernelGGL((state_bf16 ? step_fused_kernel<128, 8, 4, uint16_t> : step_fused_kernel<128, 8, 4, float>),
                               grid, block, lds, stream, sa, ca);
        else
            hipLaunchKernelGGL((state_bf16 ? step_fused_kernel<128, 16, 4, uint16_t> : step_fused_kernel<128, 16, 4, float>),
                               grid, block, lds, stream, sa, ca);
        return hipGetLastError();
    }
    hipError_t e = in_bf16 ? launch_address<true>(sa, dh, stream) : launch_address<false>(sa, dh, stream);
    if (e != hipSuccess)
        return e;
    if (state_bf16) {
        if (in_bf16)
            hipLaunchKernelGGL((step_scan_kernel<uint16_t, uint16_t>), grid, block, 0, stream, ca);
        else
            hipLaunchKernelGGL((step_scan_kernel<uint16_t, float>), grid, block, 0, stream, ca);
    } else {
        if (in_bf16)
            hipLaunchKernelGGL((step_scan_kernel<float, uint16_t>), grid, block, 0, stream, ca);
        else
            hipLaunchKernelGGL((step_scan_kernel<float, float>), grid, block, 0, stream, ca);
    }
    return hipGetLastError();
}

} // namespace sdm
