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

namespace sdm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kWaves = 4;

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
// loading its operands once and using them for all RB row tiles.
template <int DH, int RB>
__global__ __launch_bounds__(kWaves * 64) void pk_score_bf16(const uint16_t* __restrict__ q,
                                                           const uint4* __restrict__ frag,
                                                           float* __restrict__ scores, Rows r, int S)
{
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
    const uint32_t row_bytes = (uint32_t)(H * 2 * S) * 4u;
    const __amdgpu_buffer_rsrc_t out = make_rsrc(scores + ((rr0 * H + h) * 2 + half) * (long)S,
                                                 (uint32_t)(valid - 1) * row_bytes + (uint32_t)S * 4u);
    for (int ct = wave; ct < ctiles; ct += kWaves) {
        bf16x8_t b[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            b[kk] = __builtin_bit_cast(bf16x8_t, fb[(ct * KSTEPS + kk) * 64]);
        const int s = ct * 32 + i;
        const uint32_t lane_off = (uint32_t)(4 * kg) * row_bytes + (uint32_t)s * 4u;
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

template <int DH>
hipError_t launch_dh(const void* q, const void* subkeys, const void* frag, float* scores, const Rows& r, int S,
                     bool in_bf16, hipStream_t stream)
{
    if (in_bf16) {
        constexpr int RB = DH <= 128 ? 4 : 2;
        const int blocks = (r.Tc + 32 * RB - 1) / (32 * RB);
        hipLaunchKernelGGL((pk_score_bf16<DH, RB>), dim3((unsigned)(blocks * r.B * r.H * 2)), dim3(kWaves * 64), 0,
                           stream, (const uint16_t*)q, (const uint4*)frag, scores, r, S);
    } else {
        const int tiles = (r.Tc + 31) / 32;
        hipLaunchKernelGGL(pk_score_f32<DH>, dim3((unsigned)(tiles * r.B * r.H * 2)), dim3(kWaves * 64), 0, stream,
                           (const float*)q, (const float*)subkeys, scores, r, S);
    }
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

hipError_t launch_pk_score(const void* q, const void* subkeys, const void* frag, float* scores, const Rows& r,
                           int S, int dh, bool in_bf16, hipStream_t stream)
{
    if (r.count() <= 0)
        return hipSuccess;
    switch (dh) {
    case 16: return launch_dh<16>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 32: return launch_dh<32>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 48: return launch_dh<48>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 64: return launch_dh<64>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 96: return launch_dh<96>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 128: return launch_dh<128>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 192: return launch_dh<192>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    case 256: return launch_dh<256>(q, subkeys, frag, scores, r, S, in_bf16, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace sdm
