// pk_score: sub-key scoring on the matrix cores.
//
// Product-key addressing scores the two halves of every query against the two
// sub-key tables (SDM blog post, caption of the figure "The SDM mechanism, end
// to end": two sub-keys, then the outer sum).  For all rows at once this is a
// dense contraction scores[r, half, s] = sum_c q[r, half*dh + c] * K[h, half, s, c],
// which runs here on MFMA: v_mfma_f32_32x32x16_bf16 for bf16 inputs and
// v_mfma_f32_32x32x2_f32 for float32 inputs, accumulating in float32.
//
// A workgroup owns 32 rows of one head and one half; its four waves walk the
// S sub-keys in 32-wide column tiles.  Each lane keeps its slice of the 32 x dh
// query tile in registers for the whole walk; sub-key tiles are read straight
// from global memory, where the tables (S*dh elements per half and head) stay
// resident in L2 across workgroups.
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
template <int DH>
__global__ __launch_bounds__(kWaves * 64) void pk_score_bf16(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ subkeys,
                                                           float* __restrict__ scores, long rows_per_head,
                                                           int H, int S)
{
    constexpr int KSTEPS = DH / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 31, kg = lane >> 5;
    const long tiles = (rows_per_head + 31) / 32;
    long bid = blockIdx.x;
    const int half = (int)(bid & 1);
    bid >>= 1;
    const long rt = bid % tiles;
    const int h = (int)(bid / tiles);
    const int dk = 2 * DH;

    const long rr = rt * 32 + i;
    bf16x8_t a[KSTEPS];
    if (rr < rows_per_head) {
        const uint16_t* qrow = q + (rr * H + h) * dk + half * DH + kg * 8;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + kk * 16);
    } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            a[kk] = bf16x8_t{};
    }
    const uint16_t* table = subkeys + ((long)h * 2 + half) * S * DH;
    const int ctiles = (S + 31) / 32;
    for (int ct = wave; ct < ctiles; ct += kWaves) {
        const int s = ct * 32 + i;
        f32x16_t acc = {};
        if (s < S) {
            const uint16_t* krow = table + (long)s * DH + kg * 8;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(krow + kk * 16);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], bf16x8_t{}, acc, 0, 0, 0);
        }
        if (s < S) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const long row = rt * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < rows_per_head)
                    scores[((row * H + h) * 2 + half) * (long)S + s] = acc[v];
            }
        }
    }
}

template <int DH>
__global__ __launch_bounds__(kWaves * 64) void pk_score_f32(const float* __restrict__ q,
                                                          const float* __restrict__ subkeys,
                                                          float* __restrict__ scores, long rows_per_head, int H,
                                                          int S)
{
    constexpr int KSTEPS = DH / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 31, kg = lane >> 5;
    const long tiles = (rows_per_head + 31) / 32;
    long bid = blockIdx.x;
    const int half = (int)(bid & 1);
    bid >>= 1;
    const long rt = bid % tiles;
    const int h = (int)(bid / tiles);
    const int dk = 2 * DH;

    const long rr = rt * 32 + i;
    float a[KSTEPS];
    if (rr < rows_per_head) {
        const float* qrow = q + (rr * H + h) * dk + half * DH + kg;
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
                const long row = rt * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
                if (row < rows_per_head)
                    scores[((row * H + h) * 2 + half) * (long)S + s] = acc[v];
            }
        }
    }
}

template <int DH>
hipError_t launch_dh(const void* q, const void* subkeys, float* scores, long rows_per_head, int H, int S,
                     bool in_bf16, hipStream_t stream)
{
    const long tiles = (rows_per_head + 31) / 32;
    dim3 grid((unsigned)(tiles * H * 2)), block(kWaves * 64);
    if (in_bf16)
        hipLaunchKernelGGL(pk_score_bf16<DH>, grid, block, 0, stream, (const uint16_t*)q,
                           (const uint16_t*)subkeys, scores, rows_per_head, H, S);
    else
        hipLaunchKernelGGL(pk_score_f32<DH>, grid, block, 0, stream, (const float*)q, (const float*)subkeys,
                           scores, rows_per_head, H, S);
    return hipGetLastError();
}

} // namespace

hipError_t launch_pk_score(const void* q, const void* subkeys, float* scores, long rows_per_head, int H, int S,
                           int dh, bool in_bf16, hipStream_t stream)
{
    switch (dh) {
    case 16: return launch_dh<16>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 32: return launch_dh<32>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 48: return launch_dh<48>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 64: return launch_dh<64>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 96: return launch_dh<96>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 128: return launch_dh<128>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 192: return launch_dh<192>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    case 256: return launch_dh<256>(q, subkeys, scores, rows_per_head, H, S, in_bf16, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace sdm
