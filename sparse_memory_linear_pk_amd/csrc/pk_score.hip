// pk_score: sub-key scoring on the matrix cores.
//
// Product-key addressing scores the two halves of every query against the two
// sub-key tables (SDM blog post, caption of the figure "The SDM mechanism, end
// to end": two sub-keys, then the outer sum).  For all rows at once this is a
// dense contraction scores[r, half, s] = sum_c q[r, half*dh + c] * K[h, half, s, c],
// which runs here on MFMA: v_mfma_f32_32x32x16_bf16 for bf16 inputs and
// v_mfma_f32_32x32x2_f32 for float32 inputs, accumulating in float32.
//
// bf16: the sub-key tables are first rearranged into MFMA operand order (one
// contiguous kilobyte per operand load); a workgroup then owns several 32-row
// query tiles of one head and half, kept in registers, and its four waves walk
// the S sub-keys in 32-wide column tiles, each operand load serving every row
// tile.  float32 (the small shapes): one 32-row tile per workgroup, sub-key
// operands read straight from the table.
#include "sdm_internal.h"

#include <cmath>

namespace sdm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kWaves = 4;
constexpr int kLinePitch = 72; // binary16 elements per row of a wave's transpose tile (64 and 16 bytes of pad)

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// the wave's LDS accesses done and visible to its lanes
__device__ __forceinline__ void pksel_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// MFMA 32x32 operand layout used below (the same for A and B, so any ordering
// of the reduction index inside a k-step cancels out): lane l supplies row or
// column (l % 32) and the reduction slice (l / 32) of the k-step.  Result: lane
// l holds column (l % 32) of rows 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.

// Sub-key tables rearranged once per call into MFMA operand order: for head h,
// half, column tile ct and k-step kk, the 64 lanes' 16-byte operands are one
// contiguous kilobyte ([h][half][ct][kk][lane]), so every operand load is
// coalesced; sub-keys past S are zero.
__global__ __launch_bounds__(256) void pk_subkey_frag(const uint16_t* __restrict__ subkeys, uint4* __restrict__ frag,
                                                     int H, int S, int dh)
{
    const int ksteps = dh / 16, ctiles = (S + 31) / 32;
    const long n = (long)H * 2 * ctiles * ksteps * 64;
    for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int lane = (int)(e % 64);
        long r = e / 64;
        const int kk = (int)(r % ksteps);
        r /= ksteps;
        const int ct = (int)(r % ctiles);
        r /= ctiles; // h * 2 + half
        const int sk = ct * 32 + (lane & 31);
        const int c0 = kk * 16 + (lane >> 5) * 8;
        frag[e] = sk < S ? *reinterpret_cast<const uint4*>(subkeys + (r * S + sk) * (long)dh + c0)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
}

// A workgroup owns RB tiles of 32 rows of one head and half; each wave keeps
// the RB query tiles in registers and walks every fourth 32-wide sub-key tile,
// loading its operands once and using them for all RB row tiles.  HALF: the
// scores are stored as binary16 (rounded to nearest even), half the bytes.
template <int DH, int RB, bool HALF>
__global__ __launch_bounds__(kWaves * 64) void pk_score_bf16(const uint16_t* __restrict__ q,
                                                           const uint4* __restrict__ frag,
                                                           void* __restrict__ scores, Rows r, int S)
{
    constexpr uint32_t ES = HALF ? 2u : 4u; // bytes per stored score
    constexpr int KSTEPS = DH / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 31, kg = lane >> 5;
    const int H = r.H;
    // blocks of RB*32 tokens never straddle two sequences, so a block's rows are
    // evenly spaced in memory
    const int blocks = (r.Tc + 32 * RB - 1) / (32 * RB);
    int bid = blockIdx.x;
    const int half = bid & 1;
    bid >>= 1;
    const int blk = bid % blocks;
    bid /= blocks;
    const int b = bid % r.B, h = bid / r.B;
    const int dk = 2 * DH;
    const int tl0 = blk * RB * 32;                       // first token of the block, within the chunk
    const int valid = min(RB * 32, r.Tc - tl0);          // tokens of the block inside the chunk
    const long rr0 = (long)b * r.Ts + r.t0 + tl0;         // its token row (b, t) over the sequences

    bf16x8_t a[RB][KSTEPS];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const int tl = t * 32 + i;
        const uint16_t* qrow = q + ((rr0 + tl) * H + h) * dk + half * DH + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a[t][kk] = tl < valid ? *reinterpret_cast<const bf16x8_t*>(qrow + kk * 16) : bf16x8_t{};
    }
    const int ctiles = (S + 31) / 32;
    const uint4* fb = frag + (long)(h * 2 + half) * ctiles * KSTEPS * 64 + lane;
    // stores through a buffer based at the block's first row that ends with
    // the last valid row's segment: a per-lane offset (sub-key column, row
    // group) plus a uniform one per row; rows past the chunk fall outside the
    // buffer and are dropped (the host keeps 128 rows below 2^31 bytes)
    const uint32_t row_bytes = (uint32_t)(H * 2 * S) * ES;
    const __amdgpu_buffer_rsrc_t out =
        make_rsrc(static_cast<char*>(scores) + (((rr0 * H + h) * 2 + half) * (long)S) * ES,
                  (uint32_t)(valid - 1) * row_bytes + (uint32_t)S * ES);
    // the next tile's operands load while this tile's products and stores go out
    bf16x8_t bn[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
        bn[kk] = wave < ctiles ? __builtin_bit_cast(bf16x8_t, fb[(wave * KSTEPS + kk) * 64]) : bf16x8_t{};
    for (int ct = wave; ct < ctiles; ct += kWaves) {
        bf16x8_t b[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            b[kk] = bn[kk];
        const int cn = ct + kWaves < ctiles ? ct + kWaves : ct; // past the last tile: this one again, unused
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            bn[kk] = __builtin_bit_cast(bf16x8_t, fb[(cn * KSTEPS + kk) * 64]);
        const int s = ct * 32 + i;
        const uint32_t lane_off = (uint32_t)(4 * kg) * row_bytes + (uint32_t)s * ES;
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            f32x16_t acc = {};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kk], b[kk], acc, 0, 0, 0);
            if (s < S) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t row_off = (uint32_t)(t * 32 + 8 * (v >> 2) + (v & 3)) * row_bytes;
                    if constexpr (HALF)
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)acc[v]), out,
                                                              lane_off, row_off, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[v]), out, lane_off, row_off, 0);
                }
            }
        }
    }
}

template <int DH>
__global__ __launch_bounds__(kWaves * 64) void pk_score_f32(const float* __restrict__ q,
                                                          const float* __restrict__ subkeys,
                                                          float* __restrict__ scores, Rows r, int S)
{
    constexpr int KSTEPS = DH / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 31, kg = lane >> 5;
    const int H = r.H;
    const int tiles = (r.Tc + 31) / 32;
    int bid = blockIdx.x;
    const int half = bid & 1;
    bid >>= 1;
    const int tile = bid % tiles;
    bid /= tiles;
    const int b = bid % r.B, h = bid / r.B;
    const int dk = 2 * DH;
    const long rr0 = (long)b * r.Ts + r.t0 + tile * 32; // token row of the tile's first row
    const int valid = min(32, r.Tc - tile * 32);

    float a[KSTEPS];
    if (i < valid) {
        const float* qrow = q + ((rr0 + i) * H + h) * dk + half * DH + kg;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a[kk] = qrow[kk * 2];
    } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a[kk] = 0.f;
    }
    const float* table = subkeys + ((long)h * 2 + half) * S * DH;
    const int ctiles = (S + 31) / 32;
    for (int ct = wave; ct < ctiles; ct += kWaves) {
        const int s = ct * 32 + i;
        f32x16_t acc = {};
        const float* krow = table + (long)(s < S ? s : 0) * DH + kg;
        const float live = s < S ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[kk], krow[kk * 2] * live, acc, 0, 0, 0);
        if (s < S) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < valid)
                    scores[(((rr0 + row) * H + h) * 2 + half) * (long)S + s] = acc[v];
            }
        }
    }
}

// Binary16 scores in whole cache lines, for S a multiple of 32: a row's two
// halves are 4 S contiguous bytes, so with both halves of its rows in one
// workgroup, tiles 2m and 2m + 1 of the row's 2 S / 32 column tiles (half
// 0's, then half 1's) are exactly the row's m-th 128-byte line.  A workgroup
// owns 64 rows (two 32-row tiles, both query halves in registers); each wave
// walks every fourth line, passes the products through its LDS tile (32 rows x
// 64 sub-keys) and stores each line with 8 lanes of 16 bytes, so every line is
// written whole, once.
// blockIdx.y picks the query set: (q0, scores0) or (q1, scores1).
template <int DH>
__global__ __launch_bounds__(kWaves * 64) void pk_score_bf16_lines(const uint16_t* __restrict__ q0,
                                                                 const uint16_t* __restrict__ q1,
                                                                 const uint4* __restrict__ frag,
                                                                 uint16_t* __restrict__ scores0,
                                                                 uint16_t* __restrict__ scores1, Rows r, int S)
{
    constexpr int KSTEPS = DH / 16, RB = 2;
    const uint16_t* q = blockIdx.y ? q1 : q0;
    uint16_t* scores = blockIdx.y ? scores1 : scores0;
    __shared__ uint16_t s_tile[kWaves][32 * kLinePitch];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 31, kg = lane >> 5;
    uint16_t* tile = s_tile[wave];
    const int H = r.H;
    const int blocks = (r.Tc + 32 * RB - 1) / (32 * RB);
    int bid = blockIdx.x;
    const int blk = bid % blocks;
    bid /= blocks;
    const int b = bid % r.B, h = bid / r.B;
    const int dk = 2 * DH;
    const int tl0 = blk * RB * 32;
    const int valid = min(RB * 32, r.Tc - tl0);
    const long rr0 = (long)b * r.Ts + r.t0 + tl0;

    bf16x8_t a[RB][2][KSTEPS];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const int tl = t * 32 + i;
        const uint16_t* qrow = q + ((rr0 + tl) * H + h) * dk + kg * 8;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                a[t][hf][kk] = tl < valid ? *reinterpret_cast<const bf16x8_t*>(qrow + hf * DH + kk * 16) : bf16x8_t{};
    }
    const int ctiles = S / 32, lines = ctiles; // 2 ctiles column tiles per row, two per line
    const uint4* fb = frag + (long)h * 2 * ctiles * KSTEPS * 64 + lane; // tile c of the row: frag tile (h, c)
    const uint32_t row_bytes = (uint32_t)(H * 4 * S);
    const __amdgpu_buffer_rsrc_t out = make_rsrc(scores + (rr0 * H + h) * 2 * (long)S,
                                                 (uint32_t)(valid - 1) * row_bytes + (uint32_t)S * 4u);
    for (int m = wave; m < lines; m += kWaves) {
        bf16x8_t b0[KSTEPS], b1[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            b0[kk] = __builtin_bit_cast(bf16x8_t, fb[((2 * m) * KSTEPS + kk) * 64]);
            b1[kk] = __builtin_bit_cast(bf16x8_t, fb[((2 * m + 1) * KSTEPS + kk) * 64]);
        }
        const int hf0 = (2 * m) / ctiles, hf1 = (2 * m + 1) / ctiles; // query half of each tile
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf0 ? a[t][1][kk] : a[t][0][kk], b0[kk], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf1 ? a[t][1][kk] : a[t][0][kk], b1[kk], acc1, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 8 * (v >> 2) + 4 * kg + (v & 3);
                tile[row * kLinePitch + i] = __builtin_bit_cast(uint16_t, (_Float16)acc0[v]);
                tile[row * kLinePitch + 32 + i] = __builtin_bit_cast(uint16_t, (_Float16)acc1[v]);
            }
            pksel_sync();
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = u * 8 + (lane >> 3), p8 = lane & 7;
                const uint4 w = *reinterpret_cast<const uint4*>(tile + row * kLinePitch + p8 * 8);
                const uint32_t off = (uint32_t)(t * 32 + row) * row_bytes + (uint32_t)m * 128u + (uint32_t)p8 * 16u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, w), out, off, 0, 0);
            }
            pksel_sync(); // the next products overwrite the tile
        }
    }
}

// Scoring fused with the candidate search of the exact selection (bf16 inputs,
// S a multiple of 32): the scores never leave the CUs.  The selection needs,
// per row and half, a set of sub-keys that holds the half's exact top k; it
// gets every sub-key whose float32 MFMA score reaches a threshold tau, as a
// bitmask, and checks on its exact rescoring that tau was low enough (at least k
// candidates exact-score at or above tau + E, E bounding |float32 - exact|);
// the check failing, or more than 64 candidates, makes it rescore the whole
// half.  So tau only steers the cost, never the result.  It is set from the
// row's query and the table's statistics: the scores of a row against a table
// have mean <q, mu> (mu the table's mean row) and, for a table with roughly
// isotropic spread sigma per coordinate, standard deviation ~ sigma |q|, and
// tau = <q, mu> + z sigma |q| with z the normal quantile that leaves about
// cand_target(k) of S above it.
//
// MFMA roles are swapped against pk_score_bf16: the sub-key tile is the A
// operand (32 sub-keys) and the queries the B operand (32 rows), so lane l
// holds the scores of query row (l % 32) against sub-keys 8 (v / 4) + 4 (l /
// 32) + (v % 4), v = 0..15, and compares them with its own row's tau.  A wave
// owns 64 rows (two B groups) of one head and half; the two waves of a
// workgroup (128 consecutive tokens of one sequence) share each sub-key tile
// through LDS, double-buffered, with each tile's global loads issued two tiles
// ahead.  The loop is software-pipelined: the products of tile c + 1 are issued
// before the comparisons of tile c, into the other of two accumulator sets, so
// the matrix cores and the vector ALUs work at once.  Registers (at most 256
// per lane) and LDS (under 43 KB per workgroup) stay within what the scan
// leaves free, so the next chunk's scoring runs beside the scan.  Record of
// (half, row): S / 32 bit words, word c for sub-keys 32 c .. 32 c + 31 (bit p
// < 16: lane group 0 with v = 15 - p; bit p >= 16: group 1 with v = 31 - p),
// then tau's bits, then zeros, padded to cand_record_dwords(S) words; records
// [2][B * Ts * H][RW].
constexpr int kCandWaves = 2;
constexpr int kCandRows = 64 * kCandWaves; // tokens per workgroup
constexpr int kCandMaxRW = 36;             // record words for S <= 1120

// The 16 comparisons of one MFMA result as bits, first score highest: bit set
// where acc[v] < tau (the sign of acc[v] - tau; the complement marks the
// candidates).
__device__ __forceinline__ uint32_t below_bits(const f32x16_t& acc, float tau)
{
    uint32_t w = 0u;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        w = __builtin_amdgcn_alignbit(w, __float_as_uint(acc[v] - tau), 31);
    return w;
}

template <int DH>
__global__ __launch_bounds__(kCandWaves * 64) void pk_score_cand(const uint16_t* __restrict__ q0,
                                                               const uint16_t* __restrict__ q1,
                                                               const uint4* __restrict__ frag,
                                                               const float* __restrict__ kstat,
                                                               uint32_t* __restrict__ rec0,
                                                               uint32_t* __restrict__ rec1, Rows r, int S, float z)
{
    constexpr int NT = kCandWaves * 64;
    constexpr int KSTEPS = DH / 16, TILE = KSTEPS * 64; // 16-byte operand pieces per sub-key tile
    static_assert(TILE % NT == 0, "a tile loads in whole rounds of the workgroup");
    constexpr int PER = TILE / NT;
    __shared__ uint4 s_a[2][TILE];
    __shared__ uint32_t s_rec[kCandWaves][64 * kCandMaxRW];
    const uint16_t* __restrict__ q = blockIdx.y ? q1 : q0;
    uint32_t* __restrict__ rec = blockIdx.y ? rec1 : rec0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = lane >> 5;
    const int tblocks = (r.Tc + kCandRows - 1) / kCandRows;
    int bid = blockIdx.x;
    const int half = bid & 1;
    bid >>= 1;
    const int tb = bid % tblocks;
    bid /= tblocks;
    const int b = bid % r.B, h = bid / r.B;
    const int H = r.H, ctiles = S / 32, RW = cand_record_dwords(S);
    const int tw = tb * kCandRows + wave * 64; // the wave's first token in the chunk

    // Sub-key tiles stream through two register sets, each tile's loads issued
    // two tiles before its store to LDS (the tables come from the last-level
    // cache or HBM, a latency of more than a tile's work).
    const uint4* fb = frag + (long)(h * 2 + half) * ctiles * TILE;
    typedef uint32_t pieces_t __attribute__((ext_vector_type(4 * PER))); // one vector value (an array ends up in scratch)
    pieces_t R0, R1;
    auto load_tile = [&](pieces_t& R, int c) {
        c = c < ctiles ? c : ctiles - 1; // past the last tile: the last one again, unused
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const uint4 x = fb[(long)c * TILE + u * NT + threadIdx.x];
            R[4 * u] = x.x;
            R[4 * u + 1] = x.y;
            R[4 * u + 2] = x.z;
            R[4 * u + 3] = x.w;
        }
    };
    auto store_tile = [&](const pieces_t& R, int buf) {
#pragma unroll
        for (int u = 0; u < PER; ++u)
            s_a[buf][u * NT + threadIdx.x] = make_uint4(R[4 * u], R[4 * u + 1], R[4 * u + 2], R[4 * u + 3]);
    };
    load_tile(R0, 0);

    // B operands: group g, lane l -> token tw + 32 g + (l % 32), k-slice l / 32
    bf16x8_t bq[2][KSTEPS];
    float tau[2];
    const float* st = kstat + (h * 2 + half) * (DH + 4); // mean row, then sigma
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int tl = tw + 32 * g + (lane & 31);
        const long row = ((long)b * r.Ts + r.t0 + tl) * H + h;
        const uint16_t* qrow = q + row * 2 * DH + half * DH + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            bq[g][kk] = tl < r.Tc ? *reinterpret_cast<const bf16x8_t*>(qrow + kk * 16) : bf16x8_t{};
    }
    store_tile(R0, 0);
    load_tile(R1, 1);
    load_tile(R0, 2);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        float sm = 0.f, sq = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const float4 m0 = *reinterpret_cast<const float4*>(st + kk * 16 + kg * 8);
            const float4 m1 = *reinterpret_cast<const float4*>(st + kk * 16 + kg * 8 + 4);
            const float mu[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)bq[g][kk][e];
                sm = fmaf(x, mu[e], sm);
                sq = fmaf(x, x, sq);
            }
        }
        sm += __shfl_xor(sm, 32);
        sq += __shfl_xor(sq, 32);
        tau[g] = sm + z * st[DH] * sqrtf(sq);
    }
    __syncthreads(); // tile 0 in s_a[0]

    // products of tile c in accumulator set c % 2 (no copies between the sets,
    // so a step never waits for the products it has just issued)
    f32x16_t A0 = {}, A1 = {}, B0 = {}, B1 = {};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s_a[0][kk * 64 + lane]);
        A0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[0][kk], A0, 0, 0, 0);
        A1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[1][kk], A1, 0, 0, 0);
    }
    uint32_t* my = s_rec[wave] + lane * RW;
    // One tile: R holds tile ct + 1, which goes to LDS (into the buffer tile ct
    // - 1 used) and is multiplied into (n0, n1); R then takes tile ct + 3; tile
    // ct's products (c0, c1) are compared meanwhile.
    auto step = [&](int ct, pieces_t& R, const f32x16_t& c0, const f32x16_t& c1, f32x16_t& n0, f32x16_t& n1) {
        const int nb = (ct + 1) & 1;
        store_tile(R, nb);
        __syncthreads();
        load_tile(R, ct + 3);
        __builtin_amdgcn_sched_barrier(0); // the loads go out here, their wait stays at the store
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, s_a[nb][lane]);
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq[0][0], f32x16_t{}, 0, 0, 0);
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq[1][0], f32x16_t{}, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < KSTEPS; ++kk) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s_a[nb][kk * 64 + lane]);
            n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[0][kk], n0, 0, 0, 0);
            n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[1][kk], n1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0); // the products of tile ct + 1 go out before the comparisons of tile ct
        const uint32_t w0 = ~below_bits(c0, tau[0]) & 0xFFFFu, w1 = ~below_bits(c1, tau[1]) & 0xFFFFu;
        // lane l < 32 keeps row l of group 0 (its own bits and lane l + 32's),
        // lane l >= 32 row l - 32 of group 1 (lane l - 32's bits and its own):
        // v_permlane32_swap exchanges w0's upper lanes with w1's lower ones
        const auto sw = __builtin_amdgcn_permlane32_swap(w0, w1, false, false);
        my[ct] = sw[0] | (sw[1] << 16);
    };
    // the register set of tile c + 1 is (c + 1) % 2; the steps run to an even
    // count with no branch between them (so the loads' waits stay counted),
    // one past the last tile repeating it into a record word that is
    // overwritten below (ctiles < RW)
    for (int ct = 0; ct < ctiles; ct += 2) {
        step(ct, R1, A0, A1, B0, B1);
        step(ct + 1, R0, B0, B1, A0, A1);
    }
    // lane l's row: token tw + l
    const int tl = tw + lane;
    if (tl < r.Tc) {
        my[ctiles] = __float_as_uint(lane < 32 ? tau[0] : tau[1]);
        for (int c = ctiles + 1; c < RW; ++c)
            my[c] = 0u;
        const long rows_all = (long)r.B * r.Ts * H;
        const long row = ((long)b * r.Ts + r.t0 + tl) * H + h;
        uint4* dst = reinterpret_cast<uint4*>(rec + ((long)half * rows_all + row) * RW);
        for (int c = 0; c < RW / 4; ++c)
            dst[c] = make_uint4(my[4 * c], my[4 * c + 1], my[4 * c + 2], my[4 * c + 3]);
    }
}

// The statistics the fused scoring sets its thresholds from, per table (h,
// half) = blockIdx.x: the mean row mu (dh floats) and sigma, the root mean
// square deviation from it over all S dh entries; [2 H][dh + 4].  Thread t sums
// column t % dh over the rows t / dh, t / dh + 1024 / dh, ...; sums and squares
// in float32 (the thresholds steer only the cost of the selection).
constexpr int kStatThreads = 1024;

__global__ __launch_bounds__(kStatThreads) void subkey_stats_kernel(const uint16_t* __restrict__ subkeys,
                                                                    float* __restrict__ kstat, int S, int dh)
{
    __shared__ float s_sum[kStatThreads], s_sq[kStatThreads];
    const uint16_t* tab = subkeys + (long)blockIdx.x * S * dh;
    float* out = kstat + (long)blockIdx.x * (dh + 4);
    const int t = threadIdx.x, phases = kStatThreads / dh, c = t % dh, p0 = t / dh;
    float sum = 0.f, sq = 0.f;
    if (p0 < phases) {
#pragma unroll 4
        for (int j = p0; j < S; j += phases) {
            const float x = __uint_as_float((uint32_t)tab[(long)j * dh + c] << 16);
            sum += x;
            sq = fmaf(x, x, sq);
        }
    }
    s_sum[t] = sum;
    s_sq[t] = sq;
    __syncthreads();
    if (t < dh) {
        float m = 0.f, m2 = 0.f;
        for (int p = 0; p < phases; ++p) {
            m += s_sum[p * dh + t];
            m2 += s_sq[p * dh + t];
        }
        m /= (float)S;
        out[t] = m;
        s_sq[t] = fmaxf(m2 / (float)S - m * m, 0.f); // the column's variance
    }
    __syncthreads();
    if (t == 0) {
        float v = 0.f;
        for (int i = 0; i < dh; ++i)
            v += s_sq[i];
        out[dh] = sqrtf(v / (float)dh);
    }
}

// The fused scoring's per-call preparation of the sub-key tables in one pass:
// workgroup t = h * 2 + half copies table t into MFMA operand order (as
// pk_subkey_frag, S a multiple of 32), and from the same loads takes its
// largest magnitude (into partial-maximum slot 0, the other slots zero, as the
// selection reduces them) and the statistics of its threshold (mean row and
// spread, as subkey_stats_kernel).  Thread t always loads the same 8 columns
// (the lane of a 16-byte operand piece and its k-step repeat every 1024
// pieces), so its column sums need no exchange until the end.
template <int DH>
__global__ __launch_bounds__(1024) void subkey_prepare_kernel(const uint16_t* __restrict__ subkeys,
                                                              uint4* __restrict__ frag, float* __restrict__ kstat,
                                                              float* __restrict__ kmax, int S)
{
    constexpr int KSTEPS = DH / 16, NTH = 1024;
    static_assert((NTH / 64) % KSTEPS == 0, "a thread's pieces keep their lane and k-step: its 8 columns are fixed");
    __shared__ float s_sum[NTH][8], s_sq[NTH][8];
    __shared__ float s_max[NTH / 64], s_var[DH];
    const int tid = threadIdx.x, t = blockIdx.x;
    const long n = (long)(S / 32) * KSTEPS * 64;
    const uint16_t* tab = subkeys + (long)t * S * DH;
    uint4* fo = frag + (long)t * n;
    float sum[8] = {}, sq[8] = {}, mx = 0.f;
    // in rounds of 8 pieces per thread, all 8 loads in flight at once (pieces past
    // the table read as zeros, which change no sum and no maximum)
    for (long e0 = tid; e0 < n; e0 += 8 * NTH) {
        uint4 xs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long e = e0 + (long)u * NTH;
            const int ln = (int)(e % 64), kk = (int)((e / 64) % KSTEPS), ct = (int)(e / (64 * KSTEPS));
            xs[u] = e < n ? *reinterpret_cast<const uint4*>(tab + (long)(ct * 32 + (ln & 31)) * DH + kk * 16 +
                                                           (ln >> 5) * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long e = e0 + (long)u * NTH;
            if (e < n)
                fo[e] = xs[u];
            const uint32_t w[4] = {xs[u].x, xs[u].y, xs[u].z, xs[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
                sum[2 * i] += lo;
                sum[2 * i + 1] += hi;
                sq[2 * i] = fmaf(lo, lo, sq[2 * i]);
                sq[2 * i + 1] = fmaf(hi, hi, sq[2 * i + 1]);
                mx = fmaxf(mx, fmaxf(fabsf(lo), fabsf(hi)));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s_sum[tid][i] = sum[i];
        s_sq[tid][i] = sq[i];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0)
        s_max[tid >> 6] = mx;
    __syncthreads();
    if (tid < DH) {
        // column c is element c % 8 of column group g = c / 8: k-step g / 2, lane half g % 2
        const int c = tid, g = c >> 3, kk = g >> 1, hb = g & 1;
        float m = 0.f, m2 = 0.f;
        for (int j = kk; j < NTH / 64; j += KSTEPS)
            for (int r = 0; r < 32; ++r) {
                const int src = j * 64 + hb * 32 + r;
                m += s_sum[src][c & 7];
                m2 += s_sq[src][c & 7];
            }
        m /= (float)S;
        kstat[(long)t * (DH + 4) + c] = m;
        s_var[c] = fmaxf(m2 / (float)S - m * m, 0.f);
    }
    __syncthreads();
    if (tid == 0) {
        float v = 0.f, m = 0.f;
        for (int i = 0; i < DH; ++i)
            v += s_var[i];
        kstat[(long)t * (DH + 4) + DH] = sqrtf(v / (float)DH);
        for (int i = 0; i < NTH / 64; ++i)
            m = fmaxf(m, s_max[i]);
        kmax[(long)t * kAbsmaxParts] = m;
    }
    if (tid > 0 && tid < kAbsmaxParts)
        kmax[(long)t * kAbsmaxParts + tid] = 0.f;
}

template <int DH>
hipError_t launch_cand_dh(const void* q0, const void* q1, const void* frag, const float* kstat, void* rec0,
                          void* rec1, int nsets, const Rows& r, int S, float z, hipStream_t stream)
{
    const int tblocks = (r.Tc + kCandRows - 1) / kCandRows;
    hipLaunchKernelGGL(pk_score_cand<DH>, dim3((unsigned)(tblocks * r.B * r.H * 2), (unsigned)nsets), dim3(64 * kCandWaves), 0,
                       stream, (const uint16_t*)q0, (const uint16_t*)q1, (const uint4*)frag,
                       kstat, (uint32_t*)rec0, (uint32_t*)rec1, r, S, z);
    return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const void* q, const void* subkeys, const void* frag, void* scores, const Rows& r, int S,
                     bool in_bf16, bool half_out, hipStream_t stream)
{
    if (in_bf16) {
        constexpr int RB = DH <= 128 ? 4 : 2;
        const int blocks = (r.Tc + 32 * RB - 1) / (32 * RB);
        const dim3 grid((unsigned)(blocks * r.B * r.H * 2));
        if (half_out && S % 32 == 0) {
            const int blocks2 = (r.Tc + 63) / 64;
            hipLaunchKernelGGL(pk_score_bf16_lines<DH>, dim3((unsigned)(blocks2 * r.B * r.H)), dim3(kWaves * 64), 0,
                               stream, (const uint16_t*)q, (const uint16_t*)q, (const uint4*)frag, (uint16_t*)scores,
                               (uint16_t*)scores, r, S);
        } else if (half_out)
            hipLaunchKernelGGL((pk_score_bf16<DH, RB, true>), grid, dim3(kWaves * 64), 0, stream, (const uint16_t*)q,
                               (const uint4*)frag, scores, r, S);
        else
            hipLaunchKernelGGL((pk_score_bf16<DH, RB, false>), grid, dim3(kWaves * 64), 0, stream, (const uint16_t*)q,
                               (const uint4*)frag, scores, r, S);
    } else {
        if (half_out)
            return hipErrorInvalidValue;
        const int tiles = (r.Tc + 31) / 32;
        hipLaunchKernelGGL(pk_score_f32<DH>, dim3((unsigned)(tiles * r.B * r.H * 2)), dim3(kWaves * 64), 0, stream,
                           (const float*)q, (const float*)subkeys, (float*)scores, r, S);
    }
    return hipGetLastError();
}

template <int DH>
hipError_t launch_pair_dh(const void* q0, const void* q1, const void* frag, void* s0, void* s1, const Rows& r, int S,
                          hipStream_t stream)
{
    const int blocks2 = (r.Tc + 63) / 64;
    hipLaunchKernelGGL(pk_score_bf16_lines<DH>, dim3((unsigned)(blocks2 * r.B * r.H), 2u), dim3(kWaves * 64), 0, stream,
                       (const uint16_t*)q0, (const uint16_t*)q1, (const uint4*)frag, (uint16_t*)s0, (uint16_t*)s1, r,
                       S);
    return hipGetLastError();
}

} // namespace

size_t pk_score_frag_bytes(int H, int S, int dh) { return (size_t)H * 2 * ((S + 31) / 32) * (dh / 16) * 1024; }

hipError_t launch_pk_subkey_frag(const void* subkeys, void* frag, int H, int S, int dh, hipStream_t stream)
{
    const long n = (long)pk_score_frag_bytes(H, S, dh) / 16;
    hipLaunchKernelGGL(pk_subkey_frag, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const uint16_t*)subkeys, (uint4*)frag, H, S, dh);
    return hipGetLastError();
}

hipError_t launch_pk_score(const void* q, const void* subkeys, const void* frag, void* scores, const Rows& r,
                           int S, int dh, bool in_bf16, bool half_out, hipStream_t stream)
{
    if (r.count() <= 0)
        return hipSuccess;
    switch (dh) {
    case 16: return launch_dh<16>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 32: return launch_dh<32>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 48: return launch_dh<48>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 64: return launch_dh<64>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 96: return launch_dh<96>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 128: return launch_dh<128>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 192: return launch_dh<192>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    case 256: return launch_dh<256>(q, subkeys, frag, scores, r, S, in_bf16, half_out, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace sdm

namespace sdm {

hipError_t launch_pk_score_pair(const void* q0, const void* q1, const void* subkeys, const void* frag, void* s0,
                                void* s1, const Rows& r, int S, int dh, bool in_bf16, hipStream_t stream)
{
    if (r.count() <= 0)
        return hipSuccess;
    if (in_bf16 && S % 32 == 0) { // the line kernel, both sets in one launch
        switch (dh) {
        case 16: return launch_pair_dh<16>(q0, q1, frag, s0, s1, r, S, stream);
        case 32: return launch_pair_dh<32>(q0, q1, frag, s0, s1, r, S, stream);
        case 48: return launch_pair_dh<48>(q0, q1, frag, s0, s1, r, S, stream);
        case 64: return launch_pair_dh<64>(q0, q1, frag, s0, s1, r, S, stream);
        case 96: return launch_pair_dh<96>(q0, q1, frag, s0, s1, r, S, stream);
        case 128: return launch_pair_dh<128>(q0, q1, frag, s0, s1, r, S, stream);
        case 192: return launch_pair_dh<192>(q0, q1, frag, s0, s1, r, S, stream);
        case 256: return launch_pair_dh<256>(q0, q1, frag, s0, s1, r, S, stream);
        default: return hipErrorInvalidValue;
        }
    }
    const hipError_t e = launch_pk_score(q0, subkeys, frag, s0, r, S, dh, in_bf16, in_bf16, stream);
    return e != hipSuccess ? e : launch_pk_score(q1, subkeys, frag, s1, r, S, dh, in_bf16, in_bf16, stream);
}

} // namespace sdm

namespace sdm {

bool pk_cand_path(int S, int dh, int k, bool in_bf16)
{
    return in_bf16 && S % 32 == 0 && S >= 128 && cand_record_dwords(S) <= kCandMaxRW && (dh == 64 || dh == 128) &&
           k <= 48 && 2 * cand_target(k) <= S;
}

size_t subkey_stats_floats(int H, int dh) { return (size_t)2 * H * (dh + 4); }

hipError_t launch_subkey_prepare(const void* subkeys, void* frag, float* kstat, float* kmax, int H, int S, int dh,
                                 hipStream_t stream)
{
    if (!pk_cand_path(S, dh, 1, true))
        return hipErrorInvalidValue;
    if (dh == 64)
        hipLaunchKernelGGL(subkey_prepare_kernel<64>, dim3((unsigned)(2 * H)), dim3(1024), 0, stream,
                           (const uint16_t*)subkeys, (uint4*)frag, kstat, kmax, S);
    else
        hipLaunchKernelGGL(subkey_prepare_kernel<128>, dim3((unsigned)(2 * H)), dim3(1024), 0, stream,
                           (const uint16_t*)subkeys, (uint4*)frag, kstat, kmax, S);
    return hipGetLastError();
}

hipError_t launch_subkey_stats(const void* subkeys, float* kstat, int H, int S, int dh, hipStream_t stream)
{
    if (dh > kStatThreads)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(subkey_stats_kernel, dim3((unsigned)(2 * H)), dim3(kStatThreads), 0, stream,
                       (const uint16_t*)subkeys, kstat, S, dh);
    return hipGetLastError();
}

float cand_quantile(int S, int k)
{
    // z with P(N(0,1) > z) = cand_target(k) / S, by bisection on erfc
    const double p = (double)cand_target(k) / (double)S;
    double lo = -8.0, hi = 8.0;
    for (int i = 0; i < 80; ++i) {
        const double mid = 0.5 * (lo + hi);
        if (0.5 * std::erfc(mid / std::sqrt(2.0)) > p)
            lo = mid;
        else
            hi = mid;
    }
    return (float)(0.5 * (lo + hi));
}

hipError_t launch_pk_score_cand(const void* q0, const void* q1, const void* frag, const float* kstat, void* rec0,
                                void* rec1, int nsets, const Rows& r, int S, int dh, int k, hipStream_t stream)
{
    if (r.count() <= 0)
        return hipSuccess;
    if (!pk_cand_path(S, dh, k, true) || nsets < 1 || nsets > 2)
        return hipErrorInvalidValue;
    const float z = cand_quantile(S, k);
    return dh == 64 ? launch_cand_dh<64>(q0, q1, frag, kstat, rec0, rec1, nsets, r, S, z, stream)
                    : launch_cand_dh<128>(q0, q1, frag, kstat, rec0, rec1, nsets, r, S, z, stream);
}

} // namespace sdm
