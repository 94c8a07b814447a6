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
//     token on the matrix cores and two of its waves select the write and the
//     read slots with the selection of pk_topk (pk_select.h).  The float32
//     scores only locate the candidates: the selection recomputes every score
//     that can reach a half's top k exactly, so the slots and weights are those
//     of the forward, whatever the order of the float32 sums.
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
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
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

// Float32 scores of the two queries of (b, h) against both sub-key tables, into
// sc[query][half][S], on the matrix cores (within the bound E of the exact
// scores that the selection relies on, as for any order of the float32 sums).
// kmax[half] receives this lane's share of max |K| of table `half` (every
// element of a table is loaded by one lane of one wave); the caller reduces
// over the lanes and waves.  float32: rows 0 (write) and 1 (read) of a 32-row
// MFMA tile whose other rows are zero, the 32 columns sub-keys.
//
// bf16: a 32-column tile of sub-keys is 32 contiguous table rows.  Each wave
// walks its tiles with D of them in flight, loaded in coalesced 16-byte pieces
// (a kilobyte per load, through a buffer resource that ends with the tile's last
// row, so pieces past the table read zeros) and passes each through its LDS
// tile buffer (rows padded by 16 bytes, so that the operand reads hit distinct
// banks) to read it back in MFMA operand order.  The A operand holds both
// queries' halves for the whole walk: rows 0 and 1 the write and read queries'
// first halves, rows 2 and 3 their second halves; a tile of table `half` keeps
// rows 2 half and 2 half + 1.  Every wave issues the same loads in the same
// order (tiles past its share read zeros), so the wait for a tile is a fixed
// count.
template <int DH> constexpr int step_tile_u4() { return 32 * (DH / 8 + 1); }

// qd (optional, bf16): also stage query (wave >> 1) as doubles into qd and leave
// the sum of |q| over its half `half_q` in *abs_q, while the first tiles load.
template <int DH, bool BF16>
__device__ void step_scores(const StepArgs& a, int bh, float* sc, int lane, int wave, float (&kmax)[2], uint4* tile,
                            double* qd = nullptr, int half_q = 0, double* abs_q = nullptr)
{
    const int h = bh % a.H, S = a.S;
    const int i = lane & 31, kg = lane >> 5;
    const int ctiles = (S + 31) / 32;
    const int dk = 2 * DH;
    if constexpr (BF16) {
        constexpr int KSTEPS = DH / 16;
        constexpr int RP = DH / 8;             // 16-byte pieces per table row
        constexpr int PITCH = RP + 1;          // LDS row pitch in pieces
        constexpr int NP = 32 * RP / 64;       // pieces per lane per tile
        constexpr int D = NP <= 8 ? 4 : 2;     // tiles in flight: at most 32 pieces per lane
        static_assert(32 * RP % 64 == 0, "whole pieces per lane");
        // the raw query elements this lane stages, loaded first
        constexpr int QE = (2 * DH + 63) / 64;
        uint32_t qraw[QE];
        if (qd) {
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(static_cast<const uint16_t*>((wave >> 1) ? a.rq : a.wq) + (long)bh * dk, (uint32_t)dk * 2u);
#pragma unroll
            for (int e = 0; e < QE; ++e)
                qraw[e] = __builtin_amdgcn_raw_buffer_load_b16(rq, (uint32_t)(e * 64 + lane) * 2u, 0, 0);
        }
        // A operand: row r < 4 is half r >> 1 of query r & 1.  With half widths a
        // multiple of 32, v_mfma_f32_16x16x32_bf16 (lane l: row or column l % 16,
        // elements 8 (l / 16) .. + 8 of a 32-wide k-step; half the cycles of the
        // 32-row form for the four rows in use), else v_mfma_f32_32x32x16_bf16
        // (lane l: row or column l % 32, elements 8 (l / 32) .. + 8 of 16).
        constexpr bool K32 = DH % 32 == 0;
        constexpr int KS32 = K32 ? DH / 32 : 1;
        const int c16 = lane & 15, g16 = lane >> 4;
        bf16x8_t qv[K32 ? 1 : KSTEPS], qv32[KS32];
        if constexpr (K32) {
            const uint16_t* q = static_cast<const uint16_t*>((c16 & 1) ? a.rq : a.wq) + (long)bh * dk +
                                (c16 >> 1) * DH + g16 * 8;
#pragma unroll
            for (int kk = 0; kk < KS32; ++kk)
                qv32[kk] = c16 < 4 ? *reinterpret_cast<const bf16x8_t*>(q + kk * 32) : bf16x8_t{};
        } else {
            const uint16_t* q = static_cast<const uint16_t*>((i & 1) ? a.rq : a.wq) + (long)bh * dk + (i >> 1) * DH +
                                kg * 8;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                qv[kk] = i < 4 ? *reinterpret_cast<const bf16x8_t*>(q + kk * 16) : bf16x8_t{};
        }
        asm volatile("" ::: "memory"); // the query loads above go out before the tiles'
        const int ntask = 2 * ctiles;
        const int M = (ntask + kWaves - 1) / kWaves; // tiles per wave, the same for every wave
        const uint16_t* tab = static_cast<const uint16_t*>(a.subkeys) + (long)h * 2 * S * DH;
        const int wv = __builtin_amdgcn_readfirstlane(wave); // uniform: the tile walk is scalar
        // the wave's tiles are wv, wv + kWaves, ...: (half, ct) of the next one to issue
        int is_half = 0, is_ct = wv;
        auto issue = [&](uint4 (&dst)[NP]) __attribute__((always_inline)) {
            const bool live = is_half < 2;
            const int rows = live ? min(32, S - is_ct * 32) : 0; // rows of the tile inside its table
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(tab + ((long)(live ? is_half : 0) * S + (long)is_ct * 32) * DH, (uint32_t)(rows * DH * 2));
#pragma unroll
            for (int u = 0; u < NP; ++u)
                dst[u] = ld128(r, (uint32_t)(u * 64 + lane) * 16u);
            is_ct += kWaves;
            if (is_ct >= ctiles) { // wave-uniform
                is_ct -= ctiles;
                ++is_half;
            }
        };
        uint4 ring[D][NP];
        static_for<D>([&](auto jc) __attribute__((always_inline)) { issue(ring[decltype(jc)::value]); });
        if (qd) {
#pragma unroll
            for (int e = 0; e < QE; ++e)
                if (e * 64 + lane < dk)
                    qd[e * 64 + lane] = (double)__uint_as_float(qraw[e] << 16);
            pksel::wave_sync_lds();
            *abs_q = pksel::abs_sum(qd + half_q * DH, DH, lane);
        }
        uint32_t km[2] = {0u, 0u};
        int half = 0, ct = wv; // the tile processed next
        for (int mb = 0; mb < M; mb += D) {
            static_for<D>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                if (half < 2) { // wave-uniform
                    uint32_t mx = 0u;
#pragma unroll
                    for (int u = 0; u < NP; ++u) {
                        const int p = u * 64 + lane;
                        mx = absmax_bf16x8(mx, __builtin_bit_cast(bf16x8_t, ring[j][u]));
                        tile[(p / RP) * PITCH + p % RP] = ring[j][u];
                    }
                    km[half] = max(km[half], max(mx & 0xFFFFu, mx >> 16));
                    pksel::wave_sync_lds();
                    if constexpr (K32) {
                        // two 16-column halves of the tile, DH / 32 k-steps each
                        bf16x8_t bv[2][KS32];
#pragma unroll
                        for (int st = 0; st < 2; ++st)
#pragma unroll
                            for (int kk = 0; kk < KS32; ++kk)
                                bv[st][kk] = __builtin_bit_cast(bf16x8_t, tile[(st * 16 + c16) * PITCH + kk * 4 + g16]);
                        pksel::wave_sync_lds(); // the next tile overwrites the buffer
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            f32x4_t acc = {};
#pragma unroll
                            for (int kk = 0; kk < KS32; ++kk)
                                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv32[kk], bv[st][kk], acc, 0, 0, 0);
                            // lane l < 16 holds column l of rows 0..3 (v = 0..3)
                            const int s = ct * 32 + st * 16 + c16;
                            if (g16 == 0 && s < S) {
                                sc[(0 * 2 + half) * S + s] = half ? acc[2] : acc[0];
                                sc[(1 * 2 + half) * S + s] = half ? acc[3] : acc[1];
                            }
                        }
                    } else {
                        bf16x8_t bv[KSTEPS];
#pragma unroll
                        for (int kk = 0; kk < KSTEPS; ++kk)
                            bv[kk] = __builtin_bit_cast(bf16x8_t, tile[i * PITCH + kk * 2 + kg]);
                        pksel::wave_sync_lds(); // the next tile overwrites the buffer
                        f32x16_t acc = {};
#pragma unroll
                        for (int kk = 0; kk < KSTEPS; ++kk)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv[kk], bv[kk], acc, 0, 0, 0);
                        // lane l < 32 holds column l of rows 0..3 (v = 0..3)
                        const int s = ct * 32 + i;
                        if (kg == 0 && s < S) {
                            sc[(0 * 2 + half) * S + s] = half ? acc[2] : acc[0];
                            sc[(1 * 2 + half) * S + s] = half ? acc[3] : acc[1];
                        }
                    }
                    ct += kWaves;
                    if (ct >= ctiles) {
                        ct -= ctiles;
                        ++half;
                    }
                }
                issue(ring[j]);
            });
        }
        wait_vmcnt<0>(); // the last tiles' loads (past the wave's share) land before the registers are reused
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
    __shared__ uint4 s_tile[kWaves][BF16 ? step_tile_u4<DH>() : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.x;
    pksel::fill_pairs(s_pairs, a.k, a.W);
    float km[2];
    step_scores<DH, BF16>(a, bh, s_sc, lane, wave, km, s_tile[wave]);
    publish_kmax(km, s_km, lane, wave);
    __syncthreads();
    if (wave < 2) { // wave 0 selects the write slots, wave 1 the read slots
        const long o = ((long)wave * a.B * a.H + bh) * a.W;
        constexpr int es = BF16 ? 2 : 4;
        pksel::stage_query<BF16>(static_cast<const char*>(wave ? a.rq : a.wq) + (size_t)bh * 2 * DH * es, s_qd[wave],
                                 2 * DH, lane);
        const pksel::Refine r0 = step_refine<DH, BF16>(a, bh, s_qd[wave], 0, s_km, lane);
        const pksel::Refine r1 = step_refine<DH, BF16>(a, bh, s_qd[wave], 1, s_km, lane);
        pksel::select_row_exact<J, R, BF16, true>(s_sc + wave * 2 * a.S, a.S, a.k, a.W, a.n_pairs, s_pairs, lane,
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
// forms bh's addressing itself (the same selection as step_address_kernel, the
// four half selections on the four waves at once, the two top-W selections on
// two of them, with the counting sorts of a wave alone on its SIMD), then scans
// its 128 bytes.  The repeated addressing runs in parallel, so it adds no
// latency.
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
    __shared__ uint4 s_tile[kWaves][step_tile_u4<DH>()];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nchunk = c.d / (128 / (int)sizeof(ST));
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int q = wave >> 1, half = wave & 1; // waves 0, 1: write query; 2, 3: read query
    pksel::fill_pairs(s_pairs, a.k, a.W);
    // the scores, with the wave's query staged as doubles and the sum of |q| over
    // its half while the first sub-key tiles are in flight
    float km[2];
    double abs_q;
    step_scores<DH, true>(a, bh, s_sc, lane, wave, km, s_tile[wave], s_qd[wave], half, &abs_q);
    publish_kmax(km, s_km, lane, wave);
    __syncthreads();
    {
        const int h = bh % a.H;
        const pksel::Refine ref{s_qd[wave] + half * DH,
                                static_cast<const char*>(a.subkeys) + (size_t)(h * 2 + half) * a.S * DH * 2, DH,
                                pksel::bound_from(abs_q, DH, kmax_of(s_km, half))};
        pksel::select_half_exact<J, true, true>(s_sc + (q * 2 + half) * a.S, a.S, a.k, lane, s_buf[wave],
                                                s_val[q][half], s_sub[q][half], ref);
    }
    __syncthreads();
    if (wave < 2)
        pksel::select_from_lists<R, true>(a.S, a.k, a.W, a.n_pairs, s_pairs, lane, s_buf[wave], s_val[wave],
                                          s_sub[wave], s_idx[wave], s_wt[wave]);
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
